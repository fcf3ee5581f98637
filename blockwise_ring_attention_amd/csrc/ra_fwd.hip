// Forward kernels of one rank's share of Ring Attention on gfx950 (MI355X).
//
// A workgroup owns a tile of the rank's query rows for one (batch, KV head) and folds
// in, round by round in ring order, the key/value tiles that some of its queries may
// see. The fold is the online softmax of "Ring Attention and Ulysses shard a sequence
// two different ways, ...", section "Ring Attention: point-to-point rotation, and an
// online softmax that never sees the whole row at once": per query row a running
// maximum, a running sum and an un-normalised output, rescaled when the maximum grows.
//
// Layout on the matrix cores (one 64-wide wavefront, v_mfma_f32_32x32x16_bf16):
//   S^T[key][query] = K[key][:] . Q[query][:]   A = K tile (LDS), B = Q^T (registers)
//   O^T[dv][query] += V^T[dv][key] P^T[key][query]
//                                                A = V^T via LDS transpose reads,
//                                                B = P^T straight from the S^T registers
// so every lane owns one query column: the row max and row sum are in-lane reductions
// plus one exchange between the two 32-lane halves, and P never leaves registers.
#include "ra_internal.h"

#include <stdint.h>

namespace ra {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr float kNegInf = -__builtin_inff();
// The running maximum used as the exponent reference is only raised when a tile's
// maximum exceeds it by more than 2^kTau (log2 units). Exponentials then stay below
// 2^kTau; numerator and denominator share the reference, so the result is unchanged.
constexpr float kTau = 8.0f;
constexpr float kLn2 = 0.693147180559945309f;

typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// ---------------------------------------------------------------- work decode
struct Tile {
  int b, g, hset;      // batch, KV head, set of hpw query heads within the group
  int row0, row_end;   // the rank's query rows [row0, row_end)
};

// Workgroup -> tile. When the (batch, KV head, head set) streams divide evenly over the
// 8 XCDs, every tile of a stream runs on one XCD (workgroups are dealt to XCDs
// round-robin), so the K/V tiles those workgroups share stay in that XCD's L2. Within an
// XCD tiles go heaviest first: the last query rows see the most keys.
__device__ inline Tile decode_tile(const FwdArgs& a) {
  const int w = blockIdx.x;
  int stream, qrank;
  if (a.xcd_map) {
    const int xcd = w & 7, k = w >> 3, spx = a.streams >> 3;
    stream = xcd + 8 * (k % spx);
    qrank = k / spx;
  } else {
    stream = w % a.streams;
    qrank = w / a.streams;
  }
  const int qt = a.qtiles - 1 - qrank;
  Tile t;
  t.hset = stream % a.hsets;
  const int bg = stream / a.hsets;
  t.g = bg % a.hkv;
  t.b = bg / a.hkv;
  const int half = qt / a.tiles_half;
  t.row0 = half * a.rows_half + (qt % a.tiles_half) * a.prow;
  t.row_end = min(t.row0 + a.prow, (half + 1) * a.rows_half);
  return t;
}

// Global position of the rank's query row t (causal only). Zigzag: rows [0, m) are
// chunk `rank`, rows [m, 2m) chunk 2c-1-rank, chunks of m tokens ("What do you do about
// long sequences and sparse models?", section "What breaks the load balance?").
__device__ inline int query_pos(const FwdArgs& a, int t) {
  if (a.zigzag) {
    const int m = a.nq >> 1;
    return t < m ? a.rank * m + t : (2 * a.c - 1 - a.rank) * m + (t - m);
  }
  return a.rank * a.nq + t;
}

// ---------------------------------------------------------------- KV tile cursor
// Walks the KV tiles a query tile needs: rounds t in [t0, t1) use block
// (rank - t) mod c; a block is one segment (contiguous/non-causal) or two (zigzag:
// its early chunk in rows [0, m), its late chunk in rows [m, 2m)). Causal: only the
// rows a query of the tile may see are visited, so fully masked tiles are skipped.
template <int BN>
struct KvCursor {
  int t, seg, r, rend, slim, pdelta, blk;
  bool valid;

  __device__ inline bool enter(const FwdArgs& a, int qhi) {
    blk = a.rank - t;
    if (blk < 0) blk += a.c;
    int r0;
    if (a.causal && a.zigzag) {
      const int m = a.nkv >> 1;
      if (seg == 0) {
        r0 = 0; slim = m; pdelta = blk * m;
      } else {
        r0 = m; slim = 2 * m; pdelta = (2 * a.c - 1 - blk) * m - m;
      }
    } else {
      r0 = 0; slim = a.nkv; pdelta = a.causal ? blk * a.nkv : 0;
    }
    rend = slim;
    if (a.causal) {
      const int lim = qhi - pdelta + 1;   // rows whose position <= qhi
      rend = max(r0, min(rend, lim));
    }
    r = r0;
    return r < rend;
  }
  __device__ inline void seek(const FwdArgs& a, int qhi) {
    const int nseg = (a.causal && a.zigzag) ? 2 : 1;
    while (t < a.t1) {
      if (enter(a, qhi)) { valid = true; return; }
      if (++seg == nseg) { seg = 0; ++t; }
    }
    valid = false;
  }
  __device__ inline void begin(const FwdArgs& a, int qhi) {
    t = a.t0; seg = 0; seek(a, qhi);
  }
  __device__ inline void next(const FwdArgs& a, int qhi) {
    r += BN;
    if (r < rend) return;
    const int nseg = (a.causal && a.zigzag) ? 2 : 1;
    if (++seg == nseg) { seg = 0; ++t; }
    seek(a, qhi);
  }
  // True when some entry of the tile may be masked: it runs past its segment, or (causal)
  // its last key lies after the tile's first query.
  __device__ inline bool needs_mask(const FwdArgs& a, int qlo) const {
    return (r + BN > slim) || (a.causal && pdelta + r + BN - 1 > qlo);
  }
  __device__ inline bool key_ok(const FwdArgs& a, int row, int qpos) const {
    return row < slim && (!a.causal || pdelta + row <= qpos);
  }
};

// v_permlane32_swap on two copies of x: afterwards lo = [x(0..31), x(0..31)] and
// hi = [x(32..63), x(32..63)], so lo op hi combines each lane with lane ^ 32. Issued as
// inline assembly: the builtin's two results get folded into one when both operands are
// the same value, which silently drops the exchange. The s_nop covers the wait states
// between a VALU write of the operands and the permlane read.
__device__ inline void halves(float x, float& lo, float& hi) {
  lo = x;
  hi = x;
  asm("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(lo), "+v"(hi));
}

__device__ inline float xhalf_max(float x) {
  float lo, hi;
  halves(x, lo, hi);
  return fmaxf(lo, hi);
}

__device__ inline float xhalf_sum(float x) {
  float lo, hi;
  halves(x, lo, hi);
  return lo + hi;
}

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---------------------------------------------------------------- bf16 kernel
template <int D, int BN>
struct Bf16Layout {
  static constexpr int KS = D * 2 + 16;   // K row stride in LDS, bytes (b128 reads conflict-free)
  static constexpr int VS = D * 2 + 64;   // V row stride in LDS, bytes (transpose reads conflict-free)
  static constexpr int KT = BN * KS;
  static constexpr int VT = BN * VS;
  static constexpr int STAGE = KT + VT;
  static constexpr int CPR = D / 8;                  // 16-byte chunks per row
  static constexpr int CPT = BN * CPR / 256;         // chunks per thread per tensor
};

template <int D, int BN>
struct Bf16Stage {
  using L = Bf16Layout<D, BN>;
  u32x4 kr[L::CPT], vr[L::CPT];

  __device__ inline void load(const __bf16* kb, const __bf16* vb, int r, int nkv, int tid) {
#pragma unroll
    for (int u = 0; u < L::CPT; ++u) {
      const int q = tid + 256 * u, row = q / L::CPR, cc = q % L::CPR;
      const size_t off = (size_t)min(r + row, nkv - 1) * D + cc * 8;
      kr[u] = *reinterpret_cast<const u32x4*>(kb + off);
      vr[u] = *reinterpret_cast<const u32x4*>(vb + off);
    }
  }
  __device__ inline void store(char* stage, int tid) {
#pragma unroll
    for (int u = 0; u < L::CPT; ++u) {
      const int q = tid + 256 * u, row = q / L::CPR, cc = q % L::CPR;
      *reinterpret_cast<u32x4*>(stage + row * L::KS + cc * 16) = kr[u];
      *reinterpret_cast<u32x4*>(stage + L::KT + row * L::VS + cc * 16) = vr[u];
    }
  }
};

__device__ inline bf16x8 to_bf16x8(const f32x16& s, int base) {
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = (__bf16)s[base + e];
  return r;
}

template <int D>
__global__ __launch_bounds__(256, 1) void fwd_bf16_kernel(FwdArgs a) {
  constexpr int BN = 64;
  using L = Bf16Layout<D, BN>;
  constexpr int NKS = D / 16;   // k-steps of QK^T
  constexpr int NDV = D / 32;   // 32-wide blocks of the value dimension
  __shared__ __attribute__((aligned(16))) char smem[2 * L::STAGE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hf = lane >> 5, col = lane & 31;
  const Tile tile = decode_tile(a);

  const __bf16* qg = static_cast<const __bf16*>(a.q);
  const __bf16* kg = static_cast<const __bf16*>(a.k);
  const __bf16* vg = static_cast<const __bf16*>(a.v);
  __bf16* og = static_cast<__bf16*>(a.out);

  // The lane's two query columns (column blocks 2*wave and 2*wave+1).
  int head[2], row[2], qpos[2];
  bool rvalid[2];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const int cb = 2 * wave + nb;
    head[nb] = tile.g * a.G + tile.hset * a.hpw + cb % a.hpw;
    row[nb] = tile.row0 + (cb / a.hpw) * 32 + col;
    rvalid[nb] = row[nb] < tile.row_end;
    qpos[nb] = a.causal ? query_pos(a, min(row[nb], tile.row_end - 1)) : 0;
  }
  const int qlo = a.causal ? query_pos(a, tile.row0) : 0;
  const int qhi = a.causal ? query_pos(a, tile.row_end - 1) : 0;

  // Q^T fragments: lane (col, hf) holds dims 16*ks + 8*hf .. +7 of its query row.
  bf16x8 qf[2][NKS];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const __bf16* qrow = qg + (((size_t)tile.b * a.hq + head[nb]) * a.nq + (rvalid[nb] ? row[nb] : 0)) * D;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      u32x4 x = *reinterpret_cast<const u32x4*>(qrow + 16 * ks + 8 * hf);
      if (!rvalid[nb]) x = u32x4{0, 0, 0, 0};
      qf[nb][ks] = __builtin_bit_cast(bf16x8, x);
    }
  }

  f32x16 o[2][NDV];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb)
#pragma unroll
    for (int dv = 0; dv < NDV; ++dv) o[nb][dv] = f32x16{};
  float mref[2] = {kNegInf, kNegInf};   // exponent reference, log2 units
  float lsum[2] = {0.f, 0.f};           // this half's share of the running sum
  const float sc = a.scale_log2;

  const size_t blk_stride = (size_t)a.B * a.hkv * a.nkv * D;
  const size_t head_off = ((size_t)tile.b * a.hkv + tile.g) * a.nkv * D;

  // Transpose-read addressing of V^T fragments (see the kernel header).
  const int g16 = lane >> 4, i4 = (lane >> 2) & 3, a4 = lane & 3;
  const int v_lane_off = (4 * (g16 >> 1) + i4) * L::VS + (16 * (g16 & 1) + 4 * a4) * 2;

  KvCursor<BN> cur;
  cur.begin(a, qhi);
  Bf16Stage<D, BN> st;
  int buf = 0;
  if (cur.valid) {
    st.load(kg + cur.blk * blk_stride + head_off, vg + cur.blk * blk_stride + head_off, cur.r, a.nkv, tid);
    st.store(smem, tid);
  }
  __syncthreads();

  while (cur.valid) {
    KvCursor<BN> nxt = cur;
    nxt.next(a, qhi);
    if (nxt.valid)
      st.load(kg + nxt.blk * blk_stride + head_off, vg + nxt.blk * blk_stride + head_off, nxt.r, a.nkv, tid);

    const char* kl = smem + buf * L::STAGE;
    const char* vl = kl + L::KT;
    const bool msk = cur.needs_mask(a, qlo);

#pragma unroll
    for (int sub = 0; sub < BN / 32; ++sub) {
      // S^T = K Q^T for 32 keys x (2 x 32) queries.
      f32x16 s[2] = {f32x16{}, f32x16{}};
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const bf16x8 ka = *reinterpret_cast<const bf16x8*>(kl + (sub * 32 + col) * L::KS + (16 * ks + 8 * hf) * 2);
        s[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[0][ks], s[0], 0, 0, 0);
        s[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[1][ks], s[1], 0, 0, 0);
      }
      if (msk) {
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int krow = cur.r + sub * 32 + 8 * (e >> 2) + 4 * hf + (e & 3);
            if (!cur.key_ok(a, krow, qpos[nb])) s[nb][e] = kNegInf;
          }
      }
      // Online softmax, one query column per lane.
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        float mx = s[nb][0];
#pragma unroll
        for (int e = 1; e < 16; ++e) mx = fmaxf(mx, s[nb][e]);
        const float mt = xhalf_max(mx) * sc;
        if (__builtin_amdgcn_ballot_w64(mt > mref[nb] + kTau)) {
          const float mn = fmaxf(mref[nb], mt);
          // 0 when only the old reference is -inf; 1 when both are (nothing seen yet)
          const float alpha = mn == kNegInf ? 1.f : fast_exp2(mref[nb] - mn);
          lsum[nb] *= alpha;
#pragma unroll
          for (int dv = 0; dv < NDV; ++dv) o[nb][dv] *= alpha;
          mref[nb] = mn;
        }
        const float nm = mref[nb] == kNegInf ? 0.f : -mref[nb];
        float ps = 0.f;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float p = fast_exp2(__builtin_fmaf(s[nb][e], sc, nm));
          s[nb][e] = p;
          ps += p;
        }
        lsum[nb] += ps;
      }
      // O^T += V^T P^T, 16 keys per step.
#pragma unroll
      for (int ss = 0; ss < 2; ++ss) {
        const bf16x8 p0 = to_bf16x8(s[0], 8 * ss);
        const bf16x8 p1 = to_bf16x8(s[1], 8 * ss);
        const char* vb = vl + (sub * 32 + 16 * ss) * L::VS + v_lane_off;
#pragma unroll
        for (int dv = 0; dv < NDV; ++dv) {
          const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vb + dv * 64));
          const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vb + 8 * L::VS + dv * 64));
          const s16x8 v8 = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
          const bf16x8 va = __builtin_bit_cast(bf16x8, v8);
          o[0][dv] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, p0, o[0][dv], 0, 0, 0);
          o[1][dv] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, p1, o[1][dv], 0, 0, 0);
        }
      }
    }

    if (nxt.valid) st.store(smem + (buf ^ 1) * L::STAGE, tid);
    __syncthreads();
    cur = nxt;
    buf ^= 1;
  }

  // Epilogue: out = O / sum, lse = ln(sum) + reference.
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const float lt = xhalf_sum(lsum[nb]);
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    if (!rvalid[nb]) continue;
    const size_t ridx = ((size_t)tile.b * a.hq + head[nb]) * a.nq + row[nb];
    __bf16* orow = og + ridx * D;
#pragma unroll
    for (int dv = 0; dv < NDV; ++dv)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        bf16x4 w;
#pragma unroll
        for (int j = 0; j < 4; ++j) w[j] = (__bf16)(o[nb][dv][4 * i + j] * inv);
        *reinterpret_cast<bf16x4*>(orow + 32 * dv + 8 * i + 4 * hf) = w;
      }
    if (a.lse != nullptr && hf == 0)
      a.lse[ridx] = lt > 0.f ? (mref[nb] + __builtin_amdgcn_logf(lt)) * kLn2 : kNegInf;
  }
}

// ---------------------------------------------------------------- fp32 kernel
// Same fold with v_mfma_f32_32x32x2f32 (fp32 in, fp32 accumulate), one column block per
// wave, K/V tiles of 32 rows in LDS. DP = head_dim rounded up to 32; dims beyond
// head_dim are zero-filled and skipped.
template <int DP>
__global__ __launch_bounds__(256, 1) void fwd_f32_kernel(FwdArgs a) {
  constexpr int BN = 32;
  constexpr int KSF = DP + 2;   // K row stride (floats): 64 distinct banks per read
  constexpr int VSF = DP + 8;   // V row stride (floats): the two halves hit disjoint banks
  __shared__ float kl[BN * KSF];
  __shared__ float vl[BN * VSF];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hf = lane >> 5, col = lane & 31;
  const int d = a.d;
  const Tile tile = decode_tile(a);
  const float* qg = static_cast<const float*>(a.q);
  const float* kg = static_cast<const float*>(a.k);
  const float* vg = static_cast<const float*>(a.v);
  float* og = static_cast<float*>(a.out);

  const int cb = wave;
  const int head = tile.g * a.G + tile.hset * a.hpw + cb % a.hpw;
  const int row = tile.row0 + (cb / a.hpw) * 32 + col;
  const bool rvalid = row < tile.row_end;
  const int qpos = a.causal ? query_pos(a, min(row, tile.row_end - 1)) : 0;
  const int qlo = a.causal ? query_pos(a, tile.row0) : 0;
  const int qhi = a.causal ? query_pos(a, tile.row_end - 1) : 0;

  float qf[DP / 2];
  const float* qrow = qg + (((size_t)tile.b * a.hq + head) * a.nq + (rvalid ? row : 0)) * d;
#pragma unroll
  for (int ks = 0; ks < DP / 2; ++ks) qf[ks] = (rvalid && 2 * ks + hf < d) ? qrow[2 * ks + hf] : 0.f;

  f32x16 o[DP / 32];
#pragma unroll
  for (int dv = 0; dv < DP / 32; ++dv) o[dv] = f32x16{};
  float mref = kNegInf, lsum = 0.f;
  const float sc = a.scale_log2;
  const size_t blk_stride = (size_t)a.B * a.hkv * a.nkv * d;
  const size_t head_off = ((size_t)tile.b * a.hkv + tile.g) * a.nkv * d;

  KvCursor<BN> cur;
  cur.begin(a, qhi);
  while (cur.valid) {
    __syncthreads();
    const float* kb = kg + cur.blk * blk_stride + head_off;
    const float* vb = vg + cur.blk * blk_stride + head_off;
    for (int idx = tid; idx < BN * DP; idx += 256) {
      const int rr = idx / DP, cx = idx % DP;
      const size_t src = (size_t)min(cur.r + rr, a.nkv - 1) * d + cx;
      kl[rr * KSF + cx] = cx < d ? kb[src] : 0.f;
      vl[rr * VSF + cx] = cx < d ? vb[src] : 0.f;
    }
    __syncthreads();

    f32x16 s = f32x16{};
#pragma unroll
    for (int ks = 0; ks < DP / 2; ++ks)
      if (2 * ks < d) s = __builtin_amdgcn_mfma_f32_32x32x2f32(kl[col * KSF + 2 * ks + hf], qf[ks], s, 0, 0, 0);
    if (cur.needs_mask(a, qlo)) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int krow = cur.r + 8 * (e >> 2) + 4 * hf + (e & 3);
        if (!cur.key_ok(a, krow, qpos)) s[e] = kNegInf;
      }
    }
    float mx = s[0];
#pragma unroll
    for (int e = 1; e < 16; ++e) mx = fmaxf(mx, s[e]);
    const float mt = xhalf_max(mx) * sc;
    if (__builtin_amdgcn_ballot_w64(mt > mref + kTau)) {
      const float mn = fmaxf(mref, mt);
      const float alpha = mn == kNegInf ? 1.f : fast_exp2(mref - mn);
      lsum *= alpha;
#pragma unroll
      for (int dv = 0; dv < DP / 32; ++dv) o[dv] *= alpha;
      mref = mn;
    }
    const float nm = mref == kNegInf ? 0.f : -mref;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const float p = fast_exp2(__builtin_fmaf(s[e], sc, nm));
      s[e] = p;
      lsum += p;
    }
#pragma unroll
    for (int dv = 0; dv < DP / 32; ++dv)
      if (32 * dv < d) {
#pragma unroll
        for (int e = 0; e < 16; ++e)
          o[dv] = __builtin_amdgcn_mfma_f32_32x32x2f32(vl[(8 * (e >> 2) + 4 * hf + (e & 3)) * VSF + 32 * dv + col],
                                                       s[e], o[dv], 0, 0, 0);
      }
    cur.next(a, qhi);
  }

  const float lt = xhalf_sum(lsum);
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  if (!rvalid) return;
  const size_t ridx = ((size_t)tile.b * a.hq + head) * a.nq + row;
  float* orow = og + ridx * d;
#pragma unroll
  for (int dv = 0; dv < DP / 32; ++dv)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c0 = 32 * dv + 8 * i + 4 * hf;
      if (c0 < d) {
        const f32x4 w = {o[dv][4 * i] * inv, o[dv][4 * i + 1] * inv, o[dv][4 * i + 2] * inv, o[dv][4 * i + 3] * inv};
        *reinterpret_cast<f32x4*>(orow + c0) = w;
      }
    }
  if (a.lse != nullptr && hf == 0)
    a.lse[ridx] = lt > 0.f ? (mref + __builtin_amdgcn_logf(lt)) * kLn2 : kNegInf;
}

}  // namespace

hipError_t launch_forward_bf16(const FwdArgs& a, int grid, hipStream_t stream) {
  if (a.d == 128)
    hipLaunchKernelGGL(fwd_bf16_kernel<128>, dim3(grid), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(fwd_bf16_kernel<64>, dim3(grid), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_forward_f32(const FwdArgs& a, int grid, hipStream_t stream) {
  const int dp = (a.d + 31) / 32 * 32;
  switch (dp) {
    case 32: hipLaunchKernelGGL(fwd_f32_kernel<32>, dim3(grid), dim3(256), 0, stream, a); break;
    case 64: hipLaunchKernelGGL(fwd_f32_kernel<64>, dim3(grid), dim3(256), 0, stream, a); break;
    case 96: hipLaunchKernelGGL(fwd_f32_kernel<96>, dim3(grid), dim3(256), 0, stream, a); break;
    default: hipLaunchKernelGGL(fwd_f32_kernel<128>, dim3(grid), dim3(256), 0, stream, a); break;
  }
  return hipGetLastError();
}

}  // namespace ra
