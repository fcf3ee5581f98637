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
// The exponent reference is a running maximum raised lazily. Exponentials are taken
// against the current reference; it is raised (to the true running maximum, with O and
// the row sum rescaled) only when the reference is unset or some exponential may exceed
// 2^kTau, so exponentials stay below 2^kTau. Numerator and denominator share the
// reference, so the result is unchanged.
constexpr float kTau = 8.0f;
constexpr float kBig = 256.0f;   // 2^kTau
constexpr float kLn2 = 0.693147180559945309f;

typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// ---------------------------------------------------------------- work decode
struct Tile {
  int b, g, hset;      // batch, KV head, set of hpw query heads within the group
  int row0, row_end;   // the rank's query rows [row0, row_end)
};

// Workgroup -> tile. When the (batch, KV head) pairs divide evenly over the 8 XCDs,
// every tile that reads one KV head runs on one XCD (workgroups are dealt to XCDs
// round-robin), so the K/V tiles those workgroups share stay in that XCD's L2. Tiles go
// heaviest first: the last query rows see the most keys.
__device__ inline Tile decode_tile(const FwdArgs& a) {
  const int w = blockIdx.x;
  int bg, hset, qrank;
  if (a.xcd_map) {
    const int xcd = w & 7, k = w >> 3, per = (a.B * a.hkv >> 3) * a.hsets;
    qrank = k / per;
    const int rem = k % per;
    hset = rem % a.hsets;
    bg = xcd + 8 * (rem / a.hsets);
  } else {
    const int stream = w % a.streams;
    qrank = w / a.streams;
    hset = stream % a.hsets;
    bg = stream / a.hsets;
  }
  const int qt = a.qtiles - 1 - qrank;
  Tile t;
  t.hset = hset;
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
  int valid;   // int, not bool: keeps the struct a plain array of words that SROA splits

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
      if (enter(a, qhi)) { valid = 1; return; }
      if (++seg == nseg) { seg = 0; ++t; }
    }
    valid = 0;
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
// Each workgroup is 4 waves, one 32-query column block per wave, and two workgroups
// share a CU: the two waves on a SIMD belong to different workgroups, so while one is
// in its softmax (VALU) the other keeps the matrix core busy, and their barriers are
// independent.
//
// K/V tiles of BN = 64 keys go straight from global memory into LDS
// (global_load_lds_dwordx4), double-buffered, so no VGPRs are spent on staging. Rows are
// 2*D bytes, unpadded; 16-byte chunks are XOR-swizzled per row so that both the K
// fragment reads (ds_read_b128, 16 rows per pass) and the V^T transpose reads
// (ds_read_b64_tr_b16, 4 rows x 4 chunks per pass) hit distinct banks.
template <int D>
struct Bf16Layout {
  static constexpr int BN = 64;
  static constexpr int ROWB = 2 * D;             // bytes per K or V row
  static constexpr int CPR = D / 8;              // 16-byte chunks per row
  static constexpr int TILE = BN * ROWB;         // bytes of one K (or V) tile
  static constexpr int STAGE = 2 * TILE;         // K tile then V tile
  static constexpr int RPL = 128 / D;            // rows per 256-byte bank line
  static constexpr int LOADS = TILE / (16 * 256);  // 16-byte loads per thread per tile
  static constexpr int NKS = D / 16;             // k-steps of QK^T
  static constexpr int NDV = D / 32;             // 32-wide blocks of the value dimension
  static __device__ inline int kswz(int row) { return (row / RPL) & (CPR - 1); }
  static __device__ inline int vswz(int row) { return 4 * ((row / RPL) & (CPR / 4 - 1)); }
};

// Issue one stage's K and V tiles (rows r .. r+BN-1 of a block) into LDS. Each wave-wide
// load fills 1 KiB of LDS contiguously (lane i -> 16 bytes at i*16), so the lane fetches
// the global chunk that belongs in that swizzled slot: `koff`/`voff` hold those per-lane
// byte offsets relative to row r, and the per-stage base is uniform. A stage that runs
// past the block's last row (only the last, ragged tile of a block) clamps rows instead.
template <int D>
struct StageLoader {
  using L = Bf16Layout<D>;
  unsigned koff[L::LOADS], voff[L::LOADS];   // unsigned: lets the loads use a scalar base
  int row[L::LOADS];
  int wave;   // wave-uniform

  __device__ inline void init(int wave_uniform, int lane) {
    wave = wave_uniform;
#pragma unroll
    for (int u = 0; u < L::LOADS; ++u) {
      const int slot = (u * 4 + wave) * 64 + lane;
      row[u] = slot / L::CPR;
      const int phys = slot % L::CPR;
      koff[u] = row[u] * L::ROWB + ((phys ^ L::kswz(row[u])) << 4);
      voff[u] = row[u] * L::ROWB + ((phys ^ L::vswz(row[u])) << 4);
    }
  }

  __device__ inline void issue(char* stage, const __bf16* kb, const __bf16* vb, int r, int nkv) const {
    const char* kr = reinterpret_cast<const char*>(kb + (size_t)r * D);
    const char* vr = reinterpret_cast<const char*>(vb + (size_t)r * D);
    if (r + L::BN <= nkv) {
#pragma unroll
      for (int u = 0; u < L::LOADS; ++u) {
        __builtin_amdgcn_global_load_lds(kr + koff[u], stage + (u * 4 + wave) * 1024, 16, 0, 0);
        __builtin_amdgcn_global_load_lds(vr + voff[u], stage + L::TILE + (u * 4 + wave) * 1024, 16, 0, 0);
      }
    } else {
#pragma unroll
      for (int u = 0; u < L::LOADS; ++u) {
        // rows past the block repeat its last row (masked out by the fold)
        const unsigned back = max(0, r + row[u] - (nkv - 1)) * L::ROWB;
        __builtin_amdgcn_global_load_lds(kr + koff[u] - back, stage + (u * 4 + wave) * 1024, 16, 0, 0);
        __builtin_amdgcn_global_load_lds(vr + voff[u] - back, stage + L::TILE + (u * 4 + wave) * 1024, 16, 0, 0);
      }
    }
  }
};

__device__ inline bf16x8 to_bf16x8(const f32x16& s, int base) {
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = (__bf16)s[base + e];
  return r;
}

// Fold the BN keys of one stage held in LDS at `cur_buf` into the running state.
template <int D>
__device__ __forceinline__ void fold_stage(
    const FwdArgs& a, const KvCursor<Bf16Layout<D>::BN> cur, const char* cur_buf, int hf, int qlo, int qpos,
    float sc, const bf16x8 (&qf)[D / 16], const int (&koff)[D / 16],
    const int (&voff)[D / 32], f32x16 (&o)[D / 32], float& mref, float& lsum) {
  using L = Bf16Layout<D>;
  constexpr int BN = L::BN, NKS = L::NKS, NDV = L::NDV;
  const char* kt = cur_buf;
  const char* vt = cur_buf + L::TILE;
  const bool msk = cur.needs_mask(a, qlo);
#pragma unroll
  for (int sub = 0; sub < BN / 32; ++sub) {
    // S^T = K Q^T for 32 keys x 32 queries.
    bf16x8 kf[NKS];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) kf[ks] = *reinterpret_cast<const bf16x8*>(kt + sub * 32 * L::ROWB + koff[ks]);
    f32x16 s = f32x16{};
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[ks], qf[ks], s, 0, 0, 0);
    if (msk) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int krow = cur.r + sub * 32 + 8 * (e >> 2) + 4 * hf + (e & 3);
        if (!cur.key_ok(a, krow, qpos)) s[e] = kNegInf;
      }
    }
    // Online softmax, one query column per lane (two halves of 16 keys each).
    // Fast path: exponentials against the current reference. Every p is positive, so a
    // half-row whose sum stays within 2^kTau has every p within 2^kTau and needs no new
    // reference. Otherwise -- a reference not yet set (-inf), or a score that passed it
    // by more than kTau -- the wave takes the row maximum, raises the reference,
    // rescales O and the sum, and recomputes p.
    f32x16 p32;
    float ps = 0.f;
    {
      const float nm = mref == kNegInf ? 0.f : -mref;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        p32[e] = fast_exp2(__builtin_fmaf(s[e], sc, nm));
        ps += p32[e];
      }
    }
    if (__builtin_amdgcn_ballot_w64(mref == kNegInf || ps > kBig)) {
      float mx = s[0];
#pragma unroll
      for (int e = 1; e < 16; ++e) mx = fmaxf(mx, s[e]);
      const float mn = fmaxf(mref, xhalf_max(mx) * sc);
      // 0 when only the old reference is -inf; 1 when both are (nothing seen yet)
      const float alpha = mn == kNegInf ? 1.f : fast_exp2(mref - mn);
      lsum *= alpha;
#pragma unroll
      for (int dv = 0; dv < NDV; ++dv) o[dv] *= alpha;
      mref = mn;
      const float nm = mref == kNegInf ? 0.f : -mref;
      ps = 0.f;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        p32[e] = fast_exp2(__builtin_fmaf(s[e], sc, nm));
        ps += p32[e];
      }
    }
    lsum += ps;
    // O^T += V^T P^T, 16 keys per step.
#pragma unroll
    for (int ss = 0; ss < 2; ++ss) {
      const bf16x8 p = to_bf16x8(p32, 8 * ss);
      const char* vb = vt + (sub * 32 + ss * 16) * L::ROWB;
#pragma unroll
      for (int dv = 0; dv < NDV; ++dv) {
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vb + voff[dv]));
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vb + 8 * L::ROWB + voff[dv]));
        const bf16x8 va = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        o[dv] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, p, o[dv], 0, 0, 0);
      }
    }
  }
}

template <int D>
__global__ __launch_bounds__(256, 2) void fwd_bf16_kernel(FwdArgs a) {
  using L = Bf16Layout<D>;
  constexpr int BN = L::BN, NKS = L::NKS, NDV = L::NDV;
  __shared__ __attribute__((aligned(1024))) char smem0[L::STAGE];
  __shared__ __attribute__((aligned(1024))) char smem1[L::STAGE];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hf = lane >> 5, col = lane & 31;
  const Tile tile = decode_tile(a);
  const __bf16* kg = static_cast<const __bf16*>(a.k);
  const __bf16* vg = static_cast<const __bf16*>(a.v);
  StageLoader<D> ld;
  ld.init(wave, lane);

  // The lane's query column: column block `wave`.
  const int head = tile.g * a.G + tile.hset * a.hpw + wave % a.hpw;
  const int row = tile.row0 + (wave / a.hpw) * 32 + col;
  const bool rvalid = row < tile.row_end;
  const int qpos = a.causal ? query_pos(a, min(row, tile.row_end - 1)) : 0;
  const int qlo = a.causal ? query_pos(a, tile.row0) : 0;
  const int qhi = a.causal ? query_pos(a, tile.row_end - 1) : 0;

  // Q^T fragments: lane (col, hf) holds dims 16*ks + 8*hf .. +7 of its query row.
  bf16x8 qf[NKS];
  {
    const __bf16* qrow = static_cast<const __bf16*>(a.q) + (((size_t)tile.b * a.hq + head) * a.nq + (rvalid ? row : 0)) * D;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      u32x4 x = *reinterpret_cast<const u32x4*>(qrow + 16 * ks + 8 * hf);
      if (!rvalid) x = u32x4{0, 0, 0, 0};
      qf[ks] = __builtin_bit_cast(bf16x8, x);
    }
  }

  // Swizzled LDS byte offsets of this lane's fragments within a tile.
  int koff[NKS];   // K fragment: row sub*32 + col, chunk 2*ks + hf
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) koff[ks] = col * L::ROWB + (((2 * ks + hf) ^ L::kswz(col)) << 4);
  int voff[NDV];   // V^T transpose read: row 4*(g/2) + i (+ 16*ss, + 8, + 32*sub)
  {
    const int g = lane >> 4, i = (lane >> 2) & 3, aa = lane & 3;
    const int vrow = 4 * (g >> 1) + i;
#pragma unroll
    for (int dv = 0; dv < NDV; ++dv) {
      const int chunk = 4 * dv + 2 * (g & 1) + (aa >> 1);
      voff[dv] = vrow * L::ROWB + ((chunk ^ L::vswz(vrow)) << 4) + (aa & 1) * 8;
    }
  }

  f32x16 o[NDV];
#pragma unroll
  for (int dv = 0; dv < NDV; ++dv) o[dv] = f32x16{};
  float mref = kNegInf;   // exponent reference, log2 units
  float lsum = 0.f;       // this half's share of the running sum
  const float sc = a.scale_log2;

  const size_t blk_stride = (size_t)a.B * a.hkv * a.nkv * D;
  const size_t head_off = ((size_t)tile.b * a.hkv + tile.g) * a.nkv * D;

  // Stages alternate between two LDS buffers. They are distinct arrays and the loop is
  // unrolled over them, so the compiler can tell one stage's reads apart from the
  // in-flight loads of the next (one shared array would make it wait for those loads
  // before every LDS read). At each step: wait for this stage's own loads and the
  // barrier (all waves' loads visible; the other buffer's old stage read by everyone),
  // start streaming the next stage, then fold this one.
  KvCursor<BN> c0, c1;
  c0.begin(a, qhi);
  if (c0.valid)
    ld.issue(smem0, kg + c0.blk * blk_stride + head_off, vg + c0.blk * blk_stride + head_off, c0.r, a.nkv);
  while (c0.valid) {
    c1 = c0;
    c1.next(a, qhi);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (c1.valid)
      ld.issue(smem1, kg + c1.blk * blk_stride + head_off, vg + c1.blk * blk_stride + head_off, c1.r, a.nkv);
    fold_stage<D>(a, c0, smem0, hf, qlo, qpos, sc, qf, koff, voff, o, mref, lsum);
    if (!c1.valid) break;
    c0 = c1;
    c0.next(a, qhi);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (c0.valid)
      ld.issue(smem0, kg + c0.blk * blk_stride + head_off, vg + c0.blk * blk_stride + head_off, c0.r, a.nkv);
    fold_stage<D>(a, c1, smem1, hf, qlo, qpos, sc, qf, koff, voff, o, mref, lsum);
  }

  // Epilogue: out = O / sum, lse = ln(sum) + reference.
  const float lt = xhalf_sum(lsum);
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  if (!rvalid) return;
  const size_t ridx = ((size_t)tile.b * a.hq + head) * a.nq + row;
  __bf16* orow = static_cast<__bf16*>(a.out) + ridx * D;
#pragma unroll
  for (int dv = 0; dv < NDV; ++dv)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      bf16x4 w;
#pragma unroll
      for (int j = 0; j < 4; ++j) w[j] = (__bf16)(o[dv][4 * i + j] * inv);
      *reinterpret_cast<bf16x4*>(orow + 32 * dv + 8 * i + 4 * hf) = w;
    }
  if (a.lse != nullptr && hf == 0) a.lse[ridx] = lt > 0.f ? (mref + __builtin_amdgcn_logf(lt)) * kLn2 : kNegInf;
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
