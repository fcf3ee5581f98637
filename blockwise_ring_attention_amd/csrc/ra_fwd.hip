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

// Design-choice ablations. The shipped library defines none of these; the build script
// compiles one extra library per switch, each computing the same result another way, so
// that the counters and times of a choice can be compared with the kernel that makes it:
//   RA_ABLATION_XCD_SCATTER  the k-th tile of XCD x reads KV head (x + k) mod 8, so every
//                            XCD streams every KV head (no L2 locality per KV head);
//   RA_ABLATION_NO_SWIZZLE   K and V rows unswizzled in LDS (bank conflicts on the reads);
//   RA_ABLATION_NO_SKIP      every KV row of every round visited, every entry masked by
//                            predicate instead of skipped (no causal tile skipping);
//   RA_ABLATION_ONE_HEAD     one query head per workgroup (no GQA head packing; ra_host.cpp);
//   RA_ABLATION_STAGE_BARRIER a workgroup barrier before every stage instead of every pair
//                            of stages.
// Diagnostic build (also made by the build script, never shipped):
//   RA_DIAG_TIMELINE         every workgroup of the bf16 kernel writes 8 words to a buffer
//                            registered with ra_diag_timeline (below): the constant 100 MHz
//                            clock at entry, after the first stage's barrier, at the end of
//                            the stage loop and after the epilogue's stores, then HW_ID,
//                            XCC_ID, the stages of the loop and the tile (row0 << 16 | KV
//                            head). Nothing else changes, so its results are the shipped
//                            kernel's.

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
constexpr float kLog2e = 1.442695040888963407f;
// Initial exponent reference of the bf16 fold: finite, far below any finite scaled score,
// so the first unmasked exponential overflows and raises the reference (see pipe_step).
constexpr float kRef0 = -1.0e30f;
// Word 3 of a raw (stride 0) buffer resource on gfx9-family parts: 32-bit data format,
// no swizzle; accesses at or past num_records bytes are out of range.
constexpr int kBufferFlags = 0x00020000;

#if defined(RA_DIAG_TIMELINE)
__device__ unsigned long long* g_timeline = nullptr;
__device__ int g_timeline_cap = 0;
__device__ __forceinline__ void timeline(int word, unsigned long long v) {
  unsigned long long* t = g_timeline;
  if (t != nullptr && threadIdx.x == 0 && (int)blockIdx.x < g_timeline_cap) t[(size_t)blockIdx.x * 8 + word] = v;
}
#define RA_TIMELINE(word, v) timeline(word, v)
#else
#define RA_TIMELINE(word, v) ((void)0)
#endif

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
#if defined(RA_ABLATION_XCD_SCATTER)
    bg = ((xcd + k) & 7) + 8 * (rem / a.hsets);
#else
    bg = xcd + 8 * (rem / a.hsets);
#endif
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
// What a query tile's cursor needs about its queries: the positions of its first and
// last row (causal) and, under the document mask, the smallest and largest first visible
// position of its rows (0 without the mask, which changes nothing).
struct QRange {
  int lo, hi;       // positions of the tile's first and last query row
  int dmin, dmax;   // min / max over the tile's rows of the document start
};

template <int BN>
struct KvCursor {
  int t, seg, r, rend, slim, pdelta, blk;
  int mrow;    // a 32-key run starting at segment row x may hold masked entries if x > mrow
  int mlow;    // ... or if x < mlow (keys before some row's document start)
  int valid;   // int, not bool: keeps the struct a plain array of words that SROA splits

  __device__ inline bool enter(const FwdArgs& a, const QRange& q) {
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
    // A run [x, x+32) needs a mask when it passes the segment's end, or (causal) when its
    // last key lies after the tile's first query, or when it starts before the document
    // start of some row. Rows before every row's document start are not visited.
    mrow = slim - 32;
    mlow = -1;
    if (a.causal) {
#if defined(RA_ABLATION_NO_SKIP)
      mrow = -1;            // every run of every row takes the per-entry mask
      mlow = 0x7fffffff;
#else
      const int lim = q.hi - pdelta + 1;   // rows whose position <= the last query's
      rend = max(r0, min(rend, lim));
      mrow = min(mrow, q.lo - pdelta - 31);
      mlow = q.dmax - pdelta;
      r0 = max(r0, q.dmin - pdelta);
#endif
    }
    r = r0;
    return r < rend;
  }
  __device__ inline void seek(const FwdArgs& a, const QRange& q) {
    const int nseg = (a.causal && a.zigzag) ? 2 : 1;
    while (t < a.t1) {
      if (enter(a, q)) { valid = 1; return; }
      if (++seg == nseg) { seg = 0; ++t; }
    }
    valid = 0;
  }
  __device__ inline void begin(const FwdArgs& a, const QRange& q) {
    t = a.t0; seg = 0; seek(a, q);
  }
  __device__ inline void next(const FwdArgs& a, const QRange& q) {
    r += BN;
    if (r < rend) return;
    const int nseg = (a.causal && a.zigzag) ? 2 : 1;
    if (++seg == nseg) { seg = 0; ++t; }
    seek(a, q);
  }
  // The key at segment row `row` is visible to the query at qpos whose document starts at
  // qds (0 without the document mask). Non-short-circuit operators: callers apply it as a
  // select (see mask_sub).
  __device__ inline bool key_ok(const FwdArgs& a, int row, int qpos, int qds) const {
    const int pos = pdelta + row;
    return (row < slim) & ((a.causal == 0) | ((pos <= qpos) & (pos >= qds)));
  }
};

// Document start of the query at global position p, clamped to [0, c*nkv]: every key
// position x lies in [0, c*nkv), so x >= start keeps its meaning, and differences with
// positions (KvCursor::enter) cannot overflow int32 whatever the caller stored.
__device__ inline int doc_start_at(const FwdArgs& a, int p) {
  return min(max(a.doc[p], 0), a.c * a.nkv);
}

// The tile's QRange: positions qlo..qhi are contiguous (a tile never straddles a zigzag
// chunk). Under the document mask every wave reduces doc_start over those positions
// (at most 4 loads per lane, once per workgroup); the reduction is wave-uniform.
__device__ inline QRange tile_range(const FwdArgs& a, int qlo, int qhi, int lane) {
  QRange q{qlo, qhi, 0, 0};
  if (a.doc != nullptr) {
    int mn = 0x7fffffff, mx = -0x7fffffff - 1;
    for (int p = qlo + lane; p <= qhi; p += 64) {
      const int v = doc_start_at(a, p);
      mn = min(mn, v);
      mx = max(mx, v);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      mn = min(mn, __shfl_xor(mn, off));
      mx = max(mx, __shfl_xor(mx, off));
    }
    q.dmin = __builtin_amdgcn_readfirstlane(mn);
    q.dmax = __builtin_amdgcn_readfirstlane(mx);
  }
  return q;
}

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

// Epilogue of one launch for one row: the launch's partial is O / lt with lse_new
// (natural log) from the row sum lt taken against the reference mref (log2 units).
// Without accumulation the row gets exactly that. With accumulation the partial is folded
// into the running (out, lse) already in memory, a result over a disjoint key set: with
// M = max(lse_old, lse_new) and weights e^(lse - M), out = (w_old out_old + w_new out_new)
// / (w_old + w_new) and lse = M + ln(w_old + w_new) ("What do you do about long sequences
// and sparse models?", section "How does attention survive being split?"). Returned as
// factors: merged out = c_old * out_old + c_new * O.
struct RowFold {
  float c_old, c_new, lse;
};

__device__ inline RowFold fold_row(bool accumulate, float lse_old, float mref, float lt) {
  const float lse_new = lt > 0.f ? (mref + __builtin_amdgcn_logf(lt)) * kLn2 : kNegInf;
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  if (!accumulate) return RowFold{0.f, inv, lse_new};
  const float m = fmaxf(lse_old, lse_new);
  if (m == kNegInf) return RowFold{0.f, 0.f, kNegInf};
  const float w_old = fast_exp2((lse_old - m) * kLog2e);
  const float w_new = fast_exp2((lse_new - m) * kLog2e);
  const float tot = w_old + w_new;
  return RowFold{w_old / tot, w_new / tot * inv, m + __builtin_amdgcn_logf(tot) * kLn2};
}

// ---------------------------------------------------------------- bf16 kernel
// A workgroup is 8 waves, one 32-query column block each, and fills a CU (two waves per
// SIMD): every K/V stage staged in LDS serves 256 query columns.
//
// K/V stages of BN = 64 keys go straight from global memory into LDS (buffer loads that
// write LDS), so no VGPRs are spent on staging. NB = 4 buffers each for K and V tiles;
// stages are folded in pairs with one workgroup barrier per pair, and each pair loads the
// K tiles of the next pair and the V tiles one stage behind them (see the kernel). Rows
// are 2*D bytes, unpadded; 16-byte chunks are
// XOR-swizzled per row so that both the K fragment reads (ds_read_b128, 16 rows per pass)
// and the V^T transpose reads (ds_read_b64_tr_b16, 4 rows x 4 chunks per pass) hit
// distinct banks.
//
// Each wave folds its keys as a software pipeline over 32-key sub-tiles: step t issues
// the MFMAs of S = K Q^T for sub-tile t+1 and of O^T += V^T P^T for sub-tile t-1, and in
// the same basic block the vector ALU computes the softmax of sub-tile t, so the matrix
// core is fed from the wave's own instruction stream while its exponentials run.
template <int D>
struct Bf16Layout {
  static constexpr int BN = 64;                  // keys per stage
  static constexpr int WAVES = 8;
  static constexpr int ROWB = 2 * D;             // bytes per K or V row
  static constexpr int CPR = D / 8;              // 16-byte chunks per row
  static constexpr int TILE = BN * ROWB;         // bytes of one K (or V) tile
  static constexpr int NB = 4;   // stage buffers: K tiles fill LDS [0, 64K), V tiles [64K, 128K) at D = 128
  static constexpr int RPL = 128 / D;            // rows per 256-byte bank line
  static constexpr int LOADS = TILE / (16 * 64 * WAVES);  // 16-byte loads per thread per tile
  static constexpr int NKS = D / 16;             // k-steps of QK^T per 32-key sub-tile
  static constexpr int NDV = D / 32;             // 32-wide blocks of the value dimension
  // V tiles follow the NB K tiles in LDS; V^T fragment offsets carry this bias (see the
  // kernel) so that a V tile address minus the bias fits the 16-bit read offset.
  static constexpr int kVBias = NB * TILE >= 65536 ? 65536 : 0;
#if defined(RA_ABLATION_NO_SWIZZLE)
  static __device__ inline int kswz(int) { return 0; }
  static __device__ inline int vswz(int) { return 0; }
#else
  static __device__ inline int kswz(int row) { return (row / RPL) & (CPR - 1); }
  static __device__ inline int vswz(int row) { return 4 * ((row / RPL) & (CPR / 4 - 1)); }
#endif
};

// Issue one stage's K and V tiles (rows r .. r+BN-1 of one (block, batch, KV head) slab)
// into LDS with buffer loads that write LDS directly (buffer_load_dwordx4 ... lds). Each
// wave-wide load fills 1 KiB of LDS contiguously (lane i -> 16 bytes at i*16), so the
// lane fetches the global chunk that belongs in that swizzled slot: `koff`/`voff` hold
// those per-lane byte offsets relative to row r, and the row offset is a scalar. A stage
// that runs past the slab's last row (only the last, ragged tile of a block) clamps rows
// instead, so every load stays inside the slab. (The buffer form, unlike the global
// one, lets the compiler count LDS reads precisely while these loads are in flight.)
template <int D>
struct StageLoader {
  using L = Bf16Layout<D>;
  unsigned koff[L::LOADS], voff[L::LOADS];
  int row[L::LOADS];
  int wave;   // wave-uniform

  __device__ inline void init(int wave_uniform, int lane) {
    wave = wave_uniform;
#pragma unroll
    for (int u = 0; u < L::LOADS; ++u) {
      const int slot = (u * L::WAVES + wave) * 64 + lane;
      row[u] = slot / L::CPR;
      const int phys = slot % L::CPR;
      koff[u] = row[u] * L::ROWB + ((phys ^ L::kswz(row[u])) << 4);
      voff[u] = row[u] * L::ROWB + ((phys ^ L::vswz(row[u])) << 4);
    }
  }

  // The loads of one stage: buffer resources of the K and V slabs (row 0 of one (block,
  // batch, KV head) slab: nkv rows of 2*D bytes, nkv * 2 * D < 2^31 is checked on the
  // host) and the per-lane byte offsets of rows r .. r+BN-1. Rows past the slab's last
  // row (only in the last, ragged tile of a block) repeat that row; the fold masks them.
  // A plan for a stage past the end of the stream (valid = false) gets empty resources,
  // so its loads are out of range and read nothing: every stage issues the same number
  // of loads, and no branch is needed around them.
  struct Plan {
    __amdgpu_buffer_rsrc_t kr, vr;
    int ko[L::LOADS], vo[L::LOADS];
  };

  __device__ inline Plan plan(const __bf16* kb, const __bf16* vb, int r, int nkv, bool valid) const {
    Plan p;
    const int bytes = valid ? nkv * L::ROWB : 0;
    p.kr = __builtin_amdgcn_make_buffer_rsrc((void*)kb, 0, bytes, kBufferFlags);
    p.vr = __builtin_amdgcn_make_buffer_rsrc((void*)vb, 0, bytes, kBufferFlags);
    const int r0 = valid ? r : 0;
    const int soff = r0 * L::ROWB, last = nkv - 1 - r0;
#pragma unroll
    for (int u = 0; u < L::LOADS; ++u) {
      const int back = max(0, row[u] - last) * L::ROWB;
      p.ko[u] = soff + (int)koff[u] - back;
      p.vo[u] = soff + (int)voff[u] - back;
    }
    return p;
  }

  __device__ inline void issue_k(const Plan& p, char* kst) const {
    typedef __attribute__((address_space(3))) void lds_void;
#pragma unroll
    for (int u = 0; u < L::LOADS; ++u)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(p.kr, (lds_void*)(kst + (u * L::WAVES + wave) * 1024), 16, p.ko[u], 0,
                                               0, 0);
  }

  __device__ inline void issue_v(const Plan& p, char* vst) const {
    typedef __attribute__((address_space(3))) void lds_void;
#pragma unroll
    for (int u = 0; u < L::LOADS; ++u)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(p.vr, (lds_void*)(vst + (u * L::WAVES + wave) * 1024), 16, p.vo[u], 0,
                                               0, 0);
  }
};

// Wait until at most STAGES stages of this thread's K/V loads are still in flight (loads
// complete in issue order; every stage issues the same number of them). STAGES = 0 waits
// for every load of the thread.
template <int D, int STAGES>
__device__ __forceinline__ void wait_stages() {
  constexpr int N = STAGES * 2 * Bf16Layout<D>::LOADS;   // loads allowed in flight
  static_assert(N < 64, "vmcnt field");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

// Workgroup barrier between phases. No instruction is scheduled across it, and the
// memory clobber keeps the compiler from moving loads or stores over it. It waits for no
// memory counter: no LDS read is in flight when a wave arrives (the step before a barrier
// reads nothing ahead), and K/V loads are waited for explicitly (wait_stages) before it.
__device__ __forceinline__ void phase_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

__device__ inline bf16x8 to_bf16x8(const f32x16& s, int base) {
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = (__bf16)s[base + e];
  return r;
}

// Rows of one stage's segment that a 32-key sub-tile covers, and what masking needs.
struct SubInfo {
  int r;        // segment row of the sub-tile's first key
  int slim;     // end of the segment's rows
  int pdelta;   // global position of segment row x is pdelta + x (causal)
  int mask;     // some entry may be masked (see KvCursor::mrow)
};

__device__ inline SubInfo sub_info(const KvCursor<64>& c, int sub) {
  const int r = c.r + 32 * sub;
  return SubInfo{r, c.slim, c.pdelta, r > c.mrow || r < c.mlow};
}

// Set masked scores of a sub-tile to -inf. Lane (col, hf) holds keys 8*(e/4) + 4*hf + e%4
// of its query at qpos, whose document starts at qds. The predicate is combined with
// non-short-circuit operators and applied as a select, so no lane-divergent branch
// writes the score registers. (Written with short-circuit operators and an if, the
// compiler's divergent-branch lowering of this loop dropped the masking store for some
// lanes; see the document-mask parity tests.)
__device__ inline void mask_sub(const FwdArgs& a, const SubInfo& si, int hf, int qpos, int qds, f32x16& s) {
  const bool causal = a.causal != 0;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const int row = si.r + 8 * (e >> 2) + 4 * hf + (e & 3);
    const int pos = si.pdelta + row;
    const bool ok = (row < si.slim) & (!causal | ((pos <= qpos) & (pos >= qds)));
    s[e] = ok ? s[e] : kNegInf;
  }
}

// One step of the per-wave pipeline over 32-key sub-tiles (t = this step's softmax one):
//   QK: sn = K Q^T for sub-tile t+1, K rows at kt (NKS MFMAs, one chain);
//   PV: O^T += V^T P^T for sub-tile t-1, V rows at vt, P^T operands pp[0..1] (keys 0-15,
//       16-31) (2*NDV MFMAs, one per value block and key half);
//   SM: e = 2^(sc * S - ref) for sub-tile t (sc_ = S^T of t) and its lane sum ps.
// Step i pairs QK k-step i with P.V product i and two (D = 128) or four (D = 64) of the
// sixteen exponentials; LDS fragment reads run kAhead products ahead of their MFMAs, also
// across steps: the last products of a step read the first fragments of the next one
// (NXK: its K fragments from kn, NXV: its V^T fragments from vn), and a step whose first
// fragments were read that way (PRK, PRV) starts on them at once. The scheduling groups
// pin the interleave. The step after a barrier reads its own fragments (the tiles are
// complete only after the barrier). A step with only its V^T fragments read ahead issues
// each P.V product before its QK k-step, so the matrix cores start while the first K
// fragments are in flight.
constexpr int kAhead = 2;

template <int D>
struct Frags {
  bf16x8 kf[D / 16];
  s16x4 vlo[D / 16], vhi[D / 16];
};

template <int D>
__device__ __forceinline__ void read_k(const char* kt, const int (&koff)[D / 16], int i, int slot, Frags<D>& f) {
  f.kf[slot] = *reinterpret_cast<const bf16x8*>(kt + koff[i]);
}

template <int D>
__device__ __forceinline__ void read_vt(const char* vt, const int (&voff)[D / 32], int i, int slot, Frags<D>& f) {
  using L = Bf16Layout<D>;
  const int dv = i % L::NDV, ss = i / L::NDV;
  const char* vb = vt - L::kVBias + ss * 16 * L::ROWB;   // voff carries +kVBias
  f.vlo[slot] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vb + voff[dv]));
  f.vhi[slot] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vb + 8 * L::ROWB + voff[dv]));
}

struct NoExtra {
  __device__ inline void operator()() const {}
};

// `extra` is issued with product 1, inside the block: a stage's first step plans its
// loads and issues the K tile there, its second step the V tile (branch-free, see
// StageLoader::Plan).
template <int D, bool QK, bool PV, bool SM, bool PRK, bool PRV, bool NXK, bool NXV, class X = NoExtra>
__device__ __forceinline__ void pipe_block(const char* kt, const char* vt, const char* kn, const char* vn,
                                           const bf16x8 (&qf)[D / 16], const int (&koff)[D / 16],
                                           const int (&voff)[D / 32], const bf16x8 (&pp)[2], f32x16 (&o)[D / 32],
                                           f32x16& sn, const f32x16& sc_, float sc, float nm, f32x16& e, float& ps,
                                           Frags<D>& f, const X& extra = X()) {
  using L = Bf16Layout<D>;
  constexpr int NKS = L::NKS, NDV = L::NDV;
  static_assert(NKS == 2 * NDV, "one P.V product per QK k-step");
  static_assert((!PRK || QK) && (!PRV || PV), "fragments read ahead for a product the step does not make");
  constexpr int EPS = 16 / NKS;                       // exponentials per step
  constexpr int READS = (QK ? 1 : 0) + (PV ? 2 : 0);  // LDS reads per step
  constexpr int NEXT = (NXK ? 1 : 0) + (NXV ? 2 : 0);
  constexpr int AHEAD = kAhead;
  constexpr bool PVFIRST = PRV && !PRK;
#pragma unroll
  for (int i = 0; i < AHEAD; ++i) {
    if (QK && !PRK) read_k<D>(kt, koff, i, i, f);
    if (PV && !PRV) read_vt<D>(vt, voff, i, i, f);
  }
  constexpr int FIRST = AHEAD * ((QK && !PRK ? 1 : 0) + (PV && !PRV ? 2 : 0));
  if (FIRST) __builtin_amdgcn_sched_group_barrier(0x100, FIRST, 0);
  if (QK) sn = f32x16{};
  ps = 0.f;
#pragma unroll
  for (int i = 0; i < NKS; ++i) {
    if (i == 1) extra();
    const int j = i + AHEAD;   // the fragment read in this product's slot of the schedule
    if (j < NKS) {
      if (QK) read_k<D>(kt, koff, j, j, f);
      if (PV) read_vt<D>(vt, voff, j, j, f);
    } else {
      if (NXK) read_k<D>(kn, koff, j - NKS, j - NKS, f);
      if (NXV) read_vt<D>(vn, voff, j - NKS, j - NKS, f);
    }
    auto pv = [&]() {
      const int dv = i % NDV, ss = i / NDV;
      const bf16x8 va = __builtin_bit_cast(bf16x8, __builtin_shufflevector(f.vlo[i], f.vhi[i], 0, 1, 2, 3, 4, 5, 6, 7));
      o[dv] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pp[ss], o[dv], 0, 0, 0);
    };
    if (PV && PVFIRST) pv();
    if (QK) sn = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.kf[i], qf[i], sn, 0, 0, 0);
    if (SM) {
#pragma unroll
      for (int k = 0; k < EPS; ++k) {
        const int x = EPS * i + k;
        e[x] = fast_exp2(__builtin_fmaf(sc_[x], sc, nm));
        ps = x == 0 ? e[x] : ps + e[x];
      }
    }
    if (PV && !PVFIRST) pv();
    if (PVFIRST) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // P.V product i
      if (SM) __builtin_amdgcn_sched_group_barrier(0x002, 3 * EPS / 2, 0);
      if (QK) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // QK k-step i
    } else {
      if (QK) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (SM) __builtin_amdgcn_sched_group_barrier(0x002, 3 * EPS / 2, 0);
      if (PV) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    }
    if (SM) __builtin_amdgcn_sched_group_barrier(0x002, 3 * EPS - 3 * EPS / 2, 0);
    if (j < NKS) {
      if (READS) __builtin_amdgcn_sched_group_barrier(0x100, READS, 0);
    } else {
      if (NEXT) __builtin_amdgcn_sched_group_barrier(0x100, NEXT, 0);
    }
  }
}

// A full pipeline step: the masking of sub-tile t (when some of its entries may be
// masked), the interleaved block, then the online-softmax update of sub-tile t and its
// P^T operands. Fast path: exponentials against the current reference. Every p is
// positive, so a lane whose 16-key sum stays within 2^kTau has every p within 2^kTau and
// needs no new reference. Otherwise -- a score that passed the reference by more than
// kTau, which includes the first unmasked score against the initial reference kRef0,
// whose exponential overflows -- the wave takes the row maximum, raises the reference,
// rescales O (which already holds the P.V products issued in this step, taken against
// the old reference) and the sum, and recomputes p. Masked scores are -inf and give 0.
template <int D, bool QK, bool PV, bool SM, bool PRK = false, bool PRV = false, bool NXK = false,
          bool NXV = false, class X = NoExtra>
__device__ __forceinline__ void pipe_step(const FwdArgs& a, const SubInfo& si, int hf, int qds, int qpos, float sc,
                                          const char* kt, const char* vt, const bf16x8 (&qf)[D / 16],
                                          const int (&koff)[D / 16], const int (&voff)[D / 32],
                                          const bf16x8 (&pp)[2], f32x16 (&o)[D / 32], f32x16& sn, f32x16& scur,
                                          bf16x8 (&pc)[2], float& mref, float& lsum, Frags<D>& f,
                                          const char* kn = nullptr, const char* vn = nullptr, const X& extra = X()) {
  constexpr int NDV = D / 32;
  if (SM && si.mask) mask_sub(a, si, hf, qpos, qds, scur);
  const float nm = -mref;
  f32x16 e;
  float ps;
  pipe_block<D, QK, PV, SM, PRK, PRV, NXK, NXV>(kt, vt, kn, vn, qf, koff, voff, pp, o, sn, scur, sc, nm, e, ps, f,
                                                extra);
  if (SM) {
    if (__builtin_amdgcn_ballot_w64(ps > kBig)) {
      float mx = scur[0];
#pragma unroll
      for (int x = 1; x < 16; ++x) mx = fmaxf(mx, scur[x]);
      // mn >= mref stays finite; alpha is 0 when the old reference was the initial one
      const float mn = fmaxf(mref, xhalf_max(mx) * sc);
      const float alpha = fast_exp2(mref - mn);
      lsum *= alpha;
#pragma unroll
      for (int dv = 0; dv < NDV; ++dv) o[dv] *= alpha;
      mref = mn;
      const float nm2 = -mref;
      ps = 0.f;
#pragma unroll
      for (int x = 0; x < 16; ++x) {
        e[x] = fast_exp2(__builtin_fmaf(scur[x], sc, nm2));
        ps += e[x];
      }
    }
    lsum += ps;
    pc[0] = to_bf16x8(e, 0);
    pc[1] = to_bf16x8(e, 8);
  }
}

template <int D>
__global__ __launch_bounds__(512, 1) void fwd_bf16_kernel(FwdArgs a) {
#if defined(RA_DIAG_TIMELINE)
  const unsigned long long t_entry = __builtin_amdgcn_s_memrealtime();
  int loop_stages = 0;
#endif
  using L = Bf16Layout<D>;
  constexpr int BN = L::BN, NKS = L::NKS, NDV = L::NDV, NB = L::NB;
  static_assert(NB == 4, "stage buffers");
  __shared__ __attribute__((aligned(1024))) char k0[L::TILE];
  __shared__ __attribute__((aligned(1024))) char k1[L::TILE];
  __shared__ __attribute__((aligned(1024))) char k2[L::TILE];
  __shared__ __attribute__((aligned(1024))) char k3[L::TILE];
  __shared__ __attribute__((aligned(1024))) char v0[L::TILE];
  __shared__ __attribute__((aligned(1024))) char v1[L::TILE];
  __shared__ __attribute__((aligned(1024))) char v2[L::TILE];
  __shared__ __attribute__((aligned(1024))) char v3[L::TILE];
  char* const kb[4] = {k0, k1, k2, k3};
  char* const vb[4] = {v0, v1, v2, v3};

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
  const QRange qr = tile_range(a, qlo, qhi, lane);
  const int qds = a.doc != nullptr ? doc_start_at(a, qpos) : 0;   // first key position the lane's query sees

  KvCursor<BN> lc, cc;   // next stage to load, stage being folded
  lc.begin(a, qr);
  cc = lc;

  // Q^T fragments: lane (col, hf) holds dims 16*ks + 8*hf .. +7 of its query row. A
  // tile with no keys to visit (in this launch's rounds) never reads them.
  bf16x8 qf[NKS];
  if (cc.valid) {
    const size_t qidx = ((size_t)tile.b * a.hq + head) * a.nq + (rvalid ? row : 0);
    const __bf16* qrow = static_cast<const __bf16*>(a.q) + qidx * D;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      u32x4 x = *reinterpret_cast<const u32x4*>(qrow + 16 * ks + 8 * hf);
      if (!rvalid) x = u32x4{0, 0, 0, 0};
      qf[ks] = __builtin_bit_cast(bf16x8, x);
    }
  }

  // Swizzled LDS byte offsets of this lane's fragments within a tile.
  int koff[NKS];   // K fragment: row col (+ 32*sub), chunk 2*ks + hf
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) koff[ks] = col * L::ROWB + (((2 * ks + hf) ^ L::kswz(col)) << 4);
  int voff[NDV];   // V^T transpose read: row 4*(g/2) + i (+ 16*ss, + 8, + 32*sub)
  {
    const int g = lane >> 4, i = (lane >> 2) & 3, aa = lane & 3;
    const int vrow = 4 * (g >> 1) + i;
#pragma unroll
    for (int dv = 0; dv < NDV; ++dv) {
      const int chunk = 4 * dv + 2 * (g & 1) + (aa >> 1);
      // Biased by kVBias, hidden from the compiler: V tiles sit above the 64 KiB reach of
      // the ds_read offset field, and with the bias in the register each read addresses
      // its tile as register + immediate instead of spending a VALU add per read.
      voff[dv] = vrow * L::ROWB + ((chunk ^ L::vswz(vrow)) << 4) + (aa & 1) * 8 + L::kVBias;
      asm volatile("" : "+v"(voff[dv]));
    }
  }

  f32x16 o[NDV];
#pragma unroll
  for (int dv = 0; dv < NDV; ++dv) o[dv] = f32x16{};
  float mref = kRef0;     // exponent reference, log2 units
  float lsum = 0.f;       // this half's share of the running sum
  const float sc = a.scale_log2;

  const size_t blk_stride = (size_t)a.B * a.hkv * a.nkv * D;
  const size_t head_off = ((size_t)tile.b * a.hkv + tile.g) * a.nkv * D;
  // K/V slab of the block being loaded, recomputed only when the block changes.
  int slab_blk = -1;
  const __bf16* kslab = kg;
  const __bf16* vslab = vg;
  auto slab_for = [&](const KvCursor<BN>& c) {
    if (c.blk != slab_blk) {
      slab_blk = c.blk;
      kslab = kg + slab_blk * blk_stride + head_off;
      vslab = vg + slab_blk * blk_stride + head_off;
    }
  };
  // Plan the loads of the next stage to load (nothing, past the end of the stream) and
  // advance the load cursor.
  auto plan_next = [&]() {
    slab_for(lc);
    const typename StageLoader<D>::Plan pl = ld.plan(kslab, vslab, lc.r, a.nkv, lc.valid != 0);
    if (lc.valid) lc.next(a, qr);
    return pl;
  };
  // The same plan without a branch (the slab address is recomputed), for use inside a
  // step; the cursor is advanced separately.
  auto plan_at = [&](const KvCursor<BN>& c) {
    const size_t off = (size_t)c.blk * blk_stride + head_off;
    return ld.plan(kg + off, vg + off, c.r, a.nkv, c.valid != 0);
  };

  // Accumulate mode: the running (out, lse) of the lane's row, read at the start of the
  // tail (Q fragments are dead by then, so the registers are free) and used by the
  // epilogue, so the read overlaps the last P.V products instead of following them.
  // The running out is bf16 like the inputs, or fp32 (out_f32), which keeps a long
  // stream of folds from accumulating bf16 rounding. `oldr` holds the lane's old elements
  // as raw bits: four fp32 words, or four bf16 values in the low two words.
  const size_t ridx = ((size_t)tile.b * a.hq + head) * a.nq + row;
  __bf16* const orow = static_cast<__bf16*>(a.out) + ridx * D;
  float* const orowf = static_cast<float*>(a.out) + ridx * D;
  u32x4 oldr[NDV][4] = {};
  float lse_old = kNegInf;
  auto read_old = [&]() {
    if (a.acc && rvalid) {
      lse_old = a.lse[ridx];
      if (a.out_f32) {
#pragma unroll
        for (int dv = 0; dv < NDV; ++dv)
#pragma unroll
          for (int i = 0; i < 4; ++i) oldr[dv][i] = *reinterpret_cast<const u32x4*>(orowf + 32 * dv + 8 * i + 4 * hf);
      } else {
#pragma unroll
        for (int dv = 0; dv < NDV; ++dv)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
            const u32x2 b = *reinterpret_cast<const u32x2*>(orow + 32 * dv + 8 * i + 4 * hf);
            oldr[dv][i] = u32x4{b[0], b[1], 0u, 0u};
          }
      }
    }
  };

  const bool cc_any = cc.valid;   // some stage is folded
  if (cc.valid) {
    // Stages run in pairs (2w, 2w+1) with one workgroup barrier, before the even stage.
    // Stage k's K tile is read by the steps of stage k (2k-1, 2k), its V tile by those of
    // stage k+1 (the P.V products lag the scores by two sub-tiles), so the pair (2w,
    // 2w+1) reads K of 2w, 2w+1 and V of 2w-1, 2w. Those are complete at its barrier:
    // every wave waits there for all its loads, issued during the previous pair. After
    // the barrier the pair issues, inside its even stage's steps, the loads of the tiles
    // the next pair reads: K of 2w+2, 2w+3 and V of 2w+1, 2w+2 (stage k's tiles in buffer
    // k % NB), into buffers the previous pair has finished with. The V tile of 2w+3 is
    // planned with its K tile but issued by the next pair (`pend`): its buffer holds V of
    // 2w-1, which this pair reads. The buffers are distinct arrays and the loop is
    // unrolled over them, so the compiler can tell a stage's reads apart from the loads
    // in flight into the other buffers. Even sub-tiles use (sA, pA), odd ones (sB, pB).
    // Every pair issues its loads, empty ones past the end of the stream (into buffers
    // nothing reads again), so the loads need no branch and can sit inside the steps.
    // The first pair (stages 0, 1) has no previous pair: the tile's start issues, besides
    // its own K0, V0 and K1, the next pair's K2, K3, V1 and V2 into the still unused
    // buffers, and waits only for the first three before stage 0 (stage 0 reads K0, and at
    // its end K1 and V0): the later four, issued last, stay in flight behind the first.
    typename StageLoader<D>::Plan pend;
    {
      const typename StageLoader<D>::Plan p0 = plan_next();
      ld.issue_k(p0, kb[0]);
      ld.issue_v(p0, vb[0]);
      const typename StageLoader<D>::Plan p1 = plan_next();
      ld.issue_k(p1, kb[1]);
      ld.issue_v(p1, vb[1]);
      const typename StageLoader<D>::Plan p2 = plan_next();
      ld.issue_k(p2, kb[2]);
      ld.issue_v(p2, vb[2]);
      pend = plan_next();
      ld.issue_k(pend, kb[3]);
    }
    f32x16 sA, sB;
    bf16x8 pA[2], pB[2];
    Frags<D> fr;   // LDS fragments in flight, read ahead across steps (see pipe_block)
    // ---- stage 0 (buffer 0): steps -1 and 0; the last two stages' loads may be in flight
    wait_stages<D, 2>();
    phase_barrier();
    RA_TIMELINE(1, __builtin_amdgcn_s_memrealtime());
    SubInfo prev = sub_info(cc, 1);
    {
      pipe_step<D, true, false, false>(a, prev, hf, qds, qpos, sc, kb[0], vb[0], qf, koff, voff, pB, o, sA, sB, pB,
                                       mref, lsum, fr);
      // ... reads the first K fragments of stage 1 and V^T fragments of stage 0 for step 1
      pipe_step<D, true, false, true, false, false, true, true>(a, sub_info(cc, 0), hf, qds, qpos, sc,
                                                                kb[0] + 32 * L::ROWB, vb[0], qf, koff, voff, pB, o,
                                                                sB, sA, pA, mref, lsum, fr, kb[1], vb[0]);
    }
    cc.next(a, qr);
    int last = 0;   // buffer of the last stage, for the tail
    if (cc.valid) {
      for (;;) {
#pragma unroll
        for (int u = 0; u < NB; ++u) {
          // ---- stage s (buffer b); prev describes sub-tile 1 of stage s - 1 (buffer bp)
          const int b = (1 + u) % NB, bp = u % NB;
          if (u % 2 == 0) {
            // odd s: no barrier; the first fragments of both steps were read ahead
#if defined(RA_ABLATION_STAGE_BARRIER)
            phase_barrier();   // design-choice ablation (see the top of this file)
#endif
            pipe_step<D, true, true, true, true, true, true, true>(a, prev, hf, qds, qpos, sc, kb[b], vb[bp], qf,
                                                                 koff, voff, pA, o, sA, sB, pB, mref, lsum, fr,
                                                                 kb[b] + 32 * L::ROWB, vb[bp] + 32 * L::ROWB);
            pipe_step<D, true, true, true, true, true>(a, sub_info(cc, 0), hf, qds, qpos, sc, kb[b] + 32 * L::ROWB,
                                                       vb[bp] + 32 * L::ROWB, qf, koff, voff, pB, o, sB, sA, pA,
                                                       mref, lsum, fr);
          } else {
            // even s: the pair's barrier; the loads of stages s+2, s+3 (V of s+1, s+2)
            wait_stages<D, 0>();
            phase_barrier();
            typename StageLoader<D>::Plan pl;
            pipe_step<D, true, true, true, false, false, true, true>(a, prev, hf, qds, qpos, sc, kb[b], vb[bp], qf,
                                                                   koff, voff, pA, o, sA, sB, pB, mref, lsum, fr,
                                                                   kb[b] + 32 * L::ROWB, vb[bp] + 32 * L::ROWB, [&] {
                                                                     ld.issue_v(pend, vb[(b + 1) % NB]);
                                                                     pl = plan_at(lc);
                                                                     ld.issue_k(pl, kb[(b + 2) % NB]);
                                                                   });
            if (lc.valid) lc.next(a, qr);
            // ... and reads the first K fragments of stage s+1 and V^T fragments of s
            pipe_step<D, true, true, true, true, true, true, true>(a, sub_info(cc, 0), hf, qds, qpos, sc,
                                                                 kb[b] + 32 * L::ROWB, vb[bp] + 32 * L::ROWB, qf,
                                                                 koff, voff, pB, o, sB, sA, pA, mref, lsum, fr,
                                                                 kb[(b + 1) % NB], vb[b], [&] {
                                                                   ld.issue_v(pl, vb[(b + 2) % NB]);
                                                                   pend = plan_at(lc);
                                                                   ld.issue_k(pend, kb[(b + 3) % NB]);
                                                                 });
            if (lc.valid) lc.next(a, qr);
          }
          prev = sub_info(cc, 1);
          cc.next(a, qr);
#if defined(RA_DIAG_TIMELINE)
          ++loop_stages;
#endif
          if (!cc.valid) {
            last = b;
            goto tail;
          }
        }
      }
    }
  tail:
    RA_TIMELINE(2, __builtin_amdgcn_s_memrealtime());
    read_old();
    // ---- after the last stage (buffer `last`): steps 2n-1 and 2n. After an even stage
    // its V tile is complete and its first fragments were read ahead; after an odd one
    // its V tile was issued during that stage's pair, so the workgroup waits for it.
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      if (b == last) {
        if (b % 2 == 0) {
          pipe_step<D, false, true, true, false, true, false, true>(a, prev, hf, qds, qpos, sc, kb[b], vb[b], qf,
                                                                    koff, voff, pA, o, sA, sB, pB, mref, lsum, fr,
                                                                    nullptr, vb[b] + 32 * L::ROWB);
        } else {
          wait_stages<D, 0>();
          phase_barrier();
          pipe_step<D, false, true, true, false, false, false, true>(a, prev, hf, qds, qpos, sc, kb[b], vb[b], qf,
                                                                     koff, voff, pA, o, sA, sB, pB, mref, lsum, fr,
                                                                     nullptr, vb[b] + 32 * L::ROWB);
        }
        pipe_step<D, false, true, false, false, true>(a, prev, hf, qds, qpos, sc, kb[b], vb[b] + 32 * L::ROWB, qf,
                                                      koff, voff, pB, o, sB, sA, pA, mref, lsum, fr);
      }
    }
    wait_stages<D, 0>();   // the empty loads past the end are done before the workgroup ends
  }

  // Epilogue: out = O / sum, lse = ln(sum) + reference, or (accumulate) those folded into
  // the running result read above. A tile that folded no stage has nothing to add: in
  // accumulate mode its rows whose running lse is finite stay exactly as they are, so
  // they are neither read nor written.
  const float lt = xhalf_sum(lsum);
#if defined(RA_DIAG_TIMELINE)
  RA_TIMELINE(0, t_entry);
  RA_TIMELINE(4, (unsigned)__builtin_amdgcn_s_getreg((31 << 11) | 4));    // HW_ID
  RA_TIMELINE(5, (unsigned)__builtin_amdgcn_s_getreg((31 << 11) | 20));   // XCC_ID
  RA_TIMELINE(6, (unsigned)loop_stages);
  RA_TIMELINE(7, ((unsigned long long)tile.row0 << 16) | (unsigned)tile.g);
#endif
  if (!rvalid) return;
  if (a.acc && !cc_any) {
    lse_old = a.lse[ridx];
    if (lse_old > kNegInf) return;
  }
  const RowFold f = fold_row(a.acc != 0, lse_old, mref, lt);
  // Rows with nothing folded yet (lse -inf) ignore out: c_old is 0 there, and the old
  // values are replaced by zeros on their bits, so a NaN cannot reach the arithmetic
  // whatever the FP flags allow.
  const bool use_old = f.c_old != 0.f;
  if (a.out_f32) {
#pragma unroll
    for (int dv = 0; dv < NDV; ++dv)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const u32x4 ob = use_old ? oldr[dv][i] : u32x4{0u, 0u, 0u, 0u};
        const f32x4 old = __builtin_bit_cast(f32x4, ob);
        f32x4 w;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) w[jj] = __builtin_fmaf(f.c_old, old[jj], f.c_new * o[dv][4 * i + jj]);
        *reinterpret_cast<f32x4*>(orowf + 32 * dv + 8 * i + 4 * hf) = w;
      }
  } else {
#pragma unroll
    for (int dv = 0; dv < NDV; ++dv)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
        const u32x2 ob = use_old ? u32x2{oldr[dv][i][0], oldr[dv][i][1]} : u32x2{0u, 0u};
        const bf16x4 old = __builtin_bit_cast(bf16x4, ob);
        bf16x4 w;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
          w[jj] = (__bf16)__builtin_fmaf(f.c_old, (float)old[jj], f.c_new * o[dv][4 * i + jj]);
        *reinterpret_cast<bf16x4*>(orow + 32 * dv + 8 * i + 4 * hf) = w;
      }
  }
  if (a.lse != nullptr && hf == 0) a.lse[ridx] = f.lse;
#if defined(RA_DIAG_TIMELINE)
  // thread 0 holds row row0 of the tile, which is never past its end, so it gets here
  // (in plain launches) once its stores are done
  __builtin_amdgcn_s_waitcnt(0);
  RA_TIMELINE(3, __builtin_amdgcn_s_memrealtime());
#endif
}

// ---------------------------------------------------------------- fp32 kernel
// Same fold with v_mfma_f32_32x32x2f32 (fp32 in, fp32 accumulate), one column block per
// wave, K/V tiles of 32 rows in LDS. DP = head_dim rounded up to 32; dims beyond
// head_dim are zero in Q and in the LDS tiles, so their products add exact zeros and
// need no test. The next tile's rows are loaded into registers (16-byte loads) while the
// current one is folded, and written to LDS once every wave is done with it.
template <int DP>
__global__ __launch_bounds__(256, 1) void fwd_f32_kernel(FwdArgs a) {
  constexpr int BN = 32;
  constexpr int KSF = DP + 2;   // K row stride (floats): 64 distinct banks per read
  constexpr int VSF = DP + 8;   // V row stride (floats): the two halves hit disjoint banks
  constexpr int C4 = DP / 4;    // 16-byte chunks of a padded row
  constexpr int PER = BN * C4 / 256;   // chunks of K (and of V) per thread per tile
  static_assert(PER * 256 == BN * C4, "whole chunks per thread");
  __shared__ __attribute__((aligned(16))) float kl[BN * KSF];
  __shared__ __attribute__((aligned(16))) float vl[BN * VSF];

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
  const QRange qr = tile_range(a, qlo, qhi, lane);
  const int qds = a.doc != nullptr ? doc_start_at(a, qpos) : 0;

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

  // Thread tid stages chunks tid + 256 j of a tile: row idx / C4, columns 4 (idx % C4)
  // .. +3 (zeros past head_dim; head_dim is a multiple of 8, so no chunk straddles it).
  // Rows past the block's end repeat its last row; the mask drops them.
  f32x4 kr[PER], vr[PER];
  auto load_tile = [&](const KvCursor<BN>& c) {
    const float* kb = kg + c.blk * blk_stride + head_off;
    const float* vb = vg + c.blk * blk_stride + head_off;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int idx = tid + 256 * j;
      const int cx = 4 * (idx % C4);
      const size_t src = (size_t)min(c.r + idx / C4, a.nkv - 1) * d + cx;
      const bool in = cx < d;
      kr[j] = in ? *reinterpret_cast<const f32x4*>(kb + src) : f32x4{0.f, 0.f, 0.f, 0.f};
      vr[j] = in ? *reinterpret_cast<const f32x4*>(vb + src) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int idx = tid + 256 * j;
      const int rr = idx / C4, cx = 4 * (idx % C4);
      // K rows start 8-byte aligned (the stride is DP + 2): two 8-byte writes
      typedef float f32x2 __attribute__((ext_vector_type(2)));
      f32x2* kd = reinterpret_cast<f32x2*>(kl + rr * KSF + cx);
      kd[0] = f32x2{kr[j][0], kr[j][1]};
      kd[1] = f32x2{kr[j][2], kr[j][3]};
      *reinterpret_cast<f32x4*>(vl + rr * VSF + cx) = vr[j];
    }
  };

  // The cursor's validity is the same in every wave (it follows the tile's query range).
  KvCursor<BN> cur;
  cur.begin(a, qr);
  if (cur.valid) {
    load_tile(cur);
    store_tile();
  }
  while (cur.valid) {
    __syncthreads();   // the tile of `cur` is in LDS
    KvCursor<BN> nxt = cur;
    nxt.next(a, qr);
    if (nxt.valid) load_tile(nxt);   // in flight while this tile is folded

    f32x16 s = f32x16{};
#pragma unroll
    for (int ks = 0; ks < DP / 2; ++ks)
      s = __builtin_amdgcn_mfma_f32_32x32x2f32(kl[col * KSF + 2 * ks + hf], qf[ks], s, 0, 0, 0);
    if (cur.r > cur.mrow || cur.r < cur.mlow) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int krow = cur.r + 8 * (e >> 2) + 4 * hf + (e & 3);
        s[e] = cur.key_ok(a, krow, qpos, qds) ? s[e] : kNegInf;
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
#pragma unroll
      for (int e = 0; e < 16; ++e)
        o[dv] = __builtin_amdgcn_mfma_f32_32x32x2f32(vl[(8 * (e >> 2) + 4 * hf + (e & 3)) * VSF + 32 * dv + col],
                                                     s[e], o[dv], 0, 0, 0);
    __syncthreads();   // every wave is done reading this tile
    if (nxt.valid) store_tile();
    cur = nxt;
  }

  const float lt = xhalf_sum(lsum);
  if (!rvalid) return;
  const size_t ridx = ((size_t)tile.b * a.hq + head) * a.nq + row;
  float* orow = og + ridx * d;
  const RowFold f = fold_row(a.acc != 0, a.acc ? a.lse[ridx] : 0.f, mref, lt);
#pragma unroll
  for (int dv = 0; dv < DP / 32; ++dv)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c0 = 32 * dv + 8 * i + 4 * hf;
      if (c0 < d) {
        f32x4* dst = reinterpret_cast<f32x4*>(orow + c0);
        // rows with nothing folded yet (lse -inf) ignore out; the choice is made on the
        // bits, so a NaN there cannot reach the arithmetic whatever the FP flags allow
        const u32x4 ob = f.c_old != 0.f ? *reinterpret_cast<const u32x4*>(dst) : u32x4{0u, 0u, 0u, 0u};
        const f32x4 old = __builtin_bit_cast(f32x4, ob);
        f32x4 w;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) w[jj] = f.c_old * old[jj] + f.c_new * o[dv][4 * i + jj];
        *dst = w;
      }
    }
  if (a.lse != nullptr && hf == 0) a.lse[ridx] = f.lse;
}

}  // namespace

hipError_t launch_forward_bf16(const FwdArgs& a, int grid, hipStream_t stream) {
  if (a.d == 128)
    hipLaunchKernelGGL(fwd_bf16_kernel<128>, dim3(grid), dim3(512), 0, stream, a);
  else
    hipLaunchKernelGGL(fwd_bf16_kernel<64>, dim3(grid), dim3(512), 0, stream, a);
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

#if defined(RA_DIAG_TIMELINE)
// Register the timeline buffer of the diagnostic build: `capacity` workgroups of 8
// 64-bit words (workgroups past it record nothing); nullptr and 0 unregister it. Not
// part of the shipped library's C ABI; the caller synchronises the device around it.
extern "C" int ra_diag_timeline(void* buf, int capacity) {
  if (capacity < 0 || (buf == nullptr) != (capacity == 0)) return -1;
  const int zero = 0;
  unsigned long long* p = static_cast<unsigned long long*>(buf);
  if (hipMemcpyToSymbol(HIP_SYMBOL(ra::g_timeline_cap), &zero, sizeof(int)) != hipSuccess ||
      hipMemcpyToSymbol(HIP_SYMBOL(ra::g_timeline), &p, sizeof(p)) != hipSuccess ||
      hipMemcpyToSymbol(HIP_SYMBOL(ra::g_timeline_cap), &capacity, sizeof(int)) != hipSuccess)
    return -5;
  return 0;
}
#endif
