// Host side of the C ABI declared in include/ra.h: argument checks, work planning and
// launches. Nothing here touches device memory; every check runs before any launch.
#include "ra.h"

#include <climits>
#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <string>

#include "ra_internal.h"

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

bool aligned(const void* p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }

// Byte ranges [a, a + na) and [b, b + nb) share a byte (empty or NULL ranges share none).
bool overlaps(const void* a, unsigned long long na, const void* b, unsigned long long nb) {
  if (a == nullptr || b == nullptr || na == 0 || nb == 0) return false;
  const unsigned long long x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

bool head_dim_supported(int dtype, int d) {
  if (dtype == RA_BF16) return d == 64 || d == 128;
  return d >= 8 && d <= 128 && d % 8 == 0;
}

// Query heads per workgroup: the largest power of two that divides G and fits the
// workgroup's column blocks. Packing the heads of one KV group into one workgroup lets
// a single K/V tile fetch from HBM serve all of them.
int heads_per_workgroup(int G, int col_blocks) {
  int h = 1;
  while (h * 2 <= col_blocks && G % (h * 2) == 0) h *= 2;
  return h;
}

}  // namespace

extern "C" const char* ra_last_error(void) { return g_last_error.c_str(); }

extern "C" int ra_version(void) { return 300; }  // 0.3.0

namespace {

// Every forward entry point: checks, work planning and the launch. `doc` is null unless a
// document mask applies (then causal); `acc` folds the result into the running (out, lse).
int forward(const void* q, const void* k_blocks, const void* v_blocks, const int* doc, void* out, float* lse,
            int batch, int hq, int hkv, int nq, int nkv, int head_dim, int c, int rank, int causal, int zigzag,
            int round_begin, int round_end, int dtype, void* stream, bool acc = false, int out_dtype = -1) {
  if (dtype != RA_BF16 && dtype != RA_F32) return fail(RA_ERR_ARG, "unknown dtype %d", dtype);
  if (out_dtype < 0) out_dtype = dtype;
  if (out_dtype != dtype && !(dtype == RA_BF16 && out_dtype == RA_F32))
    return fail(RA_ERR_ARG, "out_dtype %d not allowed with dtype %d", out_dtype, dtype);
  if (batch < 0 || nq < 0 || nkv < 0) return fail(RA_ERR_ARG, "negative size (batch=%d nq=%d nkv=%d)", batch, nq, nkv);
  if (hq < 1 || hkv < 1) return fail(RA_ERR_ARG, "hq=%d and hkv=%d must be >= 1", hq, hkv);
  if (hq % hkv != 0) return fail(RA_ERR_ARG, "hq=%d is not a multiple of hkv=%d", hq, hkv);
  if (c < 1) return fail(RA_ERR_ARG, "c=%d must be >= 1", c);
  if (rank < 0 || rank >= c) return fail(RA_ERR_ARG, "rank=%d outside [0, %d)", rank, c);
  if (round_begin < 0 || round_end < round_begin || round_end > c)
    return fail(RA_ERR_ARG, "round range [%d, %d) outside [0, %d]", round_begin, round_end, c);
  if (!head_dim_supported(dtype, head_dim))
    return fail(RA_ERR_UNSUPPORTED, "head_dim=%d not built for %s", head_dim, dtype == RA_BF16 ? "bf16" : "fp32");
  const bool is_causal = causal != 0;
  const bool is_zigzag = is_causal && zigzag != 0;   // positions only matter under the mask
  if (is_causal && nq != nkv) return fail(RA_ERR_SHAPE, "causal needs nq == nkv (got %d, %d)", nq, nkv);
  if (is_zigzag && nkv % 2 != 0) return fail(RA_ERR_SHAPE, "zigzag needs an even nkv (got %d)", nkv);
  // Global positions (c * nkv tokens) and tile arithmetic stay in int32.
  if ((long long)c * nkv > INT_MAX / 2) return fail(RA_ERR_SHAPE, "sequence c*nkv=%lld too long", (long long)c * nkv);
  // One (block, batch, KV head) slab of K or V is addressed with 32-bit byte offsets.
  const long long elem_bytes = dtype == RA_BF16 ? 2 : 4;
  if ((long long)nkv * head_dim * elem_bytes > INT_MAX)
    return fail(RA_ERR_SHAPE, "nkv=%d rows of head_dim=%d exceed 2 GiB per KV head slab", nkv, head_dim);
  if (batch == 0 || nq == 0) return RA_OK;

  if (q == nullptr || out == nullptr) return fail(RA_ERR_ARG, "q and out must not be NULL");
  if (nkv > 0 && (k_blocks == nullptr || v_blocks == nullptr))
    return fail(RA_ERR_ARG, "k_blocks and v_blocks must not be NULL");
  if (!aligned(q, 16) || !aligned(out, 16) || !aligned(k_blocks, 16) || !aligned(v_blocks, 16))
    return fail(RA_ERR_ALIGN, "q, k_blocks, v_blocks and out must be 16-byte aligned");
  if (!aligned(lse, 4)) return fail(RA_ERR_ALIGN, "lse must be 4-byte aligned");
  if (!aligned(doc, 4)) return fail(RA_ERR_ALIGN, "doc_start must be 4-byte aligned");
  if (acc && lse == nullptr) return fail(RA_ERR_ARG, "accumulating needs the running lse (got NULL)");
  {
    // The kernels read q, k, v and doc_start while they write out and lse.
    const unsigned long long rows = (unsigned long long)batch * hq * nq;
    const unsigned long long q_bytes = rows * head_dim * elem_bytes;
    const unsigned long long kv_bytes = (unsigned long long)c * batch * hkv * nkv * head_dim * elem_bytes;
    const unsigned long long out_bytes = rows * head_dim * (out_dtype == RA_F32 ? 4 : 2);
    const unsigned long long lse_bytes = lse != nullptr ? rows * 4 : 0;
    const unsigned long long doc_bytes = doc != nullptr ? (unsigned long long)c * nkv * 4 : 0;
    const void* in[4] = {q, k_blocks, v_blocks, doc};
    const unsigned long long in_bytes[4] = {q_bytes, kv_bytes, kv_bytes, doc_bytes};
    for (int i = 0; i < 4; ++i) {
      if (overlaps(out, out_bytes, in[i], in_bytes[i]) || overlaps(lse, lse_bytes, in[i], in_bytes[i]))
        return fail(RA_ERR_ARG, "out and lse must not overlap q, k_blocks, v_blocks or doc_start");
    }
    if (overlaps(out, out_bytes, lse, lse_bytes)) return fail(RA_ERR_ARG, "out and lse must not overlap");
  }

  ra::FwdArgs a{};
  a.q = q; a.k = k_blocks; a.v = v_blocks; a.out = out; a.lse = lse; a.doc = doc; a.acc = acc ? 1 : 0;
  a.out_f32 = (dtype == RA_BF16 && out_dtype == RA_F32) ? 1 : 0;
  a.B = batch; a.hq = hq; a.hkv = hkv; a.nq = nq; a.nkv = nkv; a.d = head_dim;
  a.c = c; a.rank = rank; a.causal = is_causal; a.zigzag = is_zigzag; a.t0 = round_begin; a.t1 = round_end;
  const int col_blocks = dtype == RA_BF16 ? ra::kBf16ColBlocks : ra::kF32ColBlocks;
  a.G = hq / hkv;
#if defined(RA_ABLATION_ONE_HEAD)
  a.hpw = dtype == RA_BF16 ? 1 : heads_per_workgroup(a.G, col_blocks);   // design-choice ablation, see ra_fwd.hip
#else
  a.hpw = heads_per_workgroup(a.G, col_blocks);
#endif
  a.hsets = a.G / a.hpw;
  a.prow = 32 * (col_blocks / a.hpw);
  a.nhalves = is_zigzag ? 2 : 1;
  a.rows_half = nq / a.nhalves;
  a.tiles_half = (a.rows_half + a.prow - 1) / a.prow;
  a.qtiles = a.nhalves * a.tiles_half;
  const long long streams = (long long)batch * hkv * a.hsets;
  const long long grid = streams * a.qtiles;
  if (grid > INT_MAX) return fail(RA_ERR_SHAPE, "too many tiles (%lld)", grid);
  a.streams = (int)streams;
  a.xcd_map = ((long long)batch * hkv) % 8 == 0;
  a.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)head_dim));

  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = dtype == RA_BF16 ? ra::launch_forward_bf16(a, (int)grid, s) : ra::launch_forward_f32(a, (int)grid, s);
  if (e != hipSuccess) return fail(RA_ERR_LAUNCH, "launch failed: %s", hipGetErrorString(e));
  return RA_OK;
}

}  // namespace

extern "C" int ra_rank_forward(const void* q, const void* k_blocks, const void* v_blocks, void* out, float* lse,
                               int batch, int hq, int hkv, int nq, int nkv, int head_dim, int c, int rank,
                               int causal, int zigzag, int round_begin, int round_end, int dtype, void* stream) {
  return forward(q, k_blocks, v_blocks, nullptr, out, lse, batch, hq, hkv, nq, nkv, head_dim, c, rank, causal,
                 zigzag, round_begin, round_end, dtype, stream);
}

extern "C" int ra_rank_forward_doc(const void* q, const void* k_blocks, const void* v_blocks, const int* doc_start,
                                   void* out, float* lse, int batch, int hq, int hkv, int nq, int nkv, int head_dim,
                                   int c, int rank, int zigzag, int round_begin, int round_end, int dtype,
                                   void* stream) {
  if (doc_start == nullptr && batch > 0 && nq > 0) return fail(RA_ERR_ARG, "doc_start must not be NULL");
  return forward(q, k_blocks, v_blocks, doc_start, out, lse, batch, hq, hkv, nq, nkv, head_dim, c, rank, 1, zigzag,
                 round_begin, round_end, dtype, stream);
}

extern "C" int ra_rank_forward_accumulate(const void* q, const void* k_blocks, const void* v_blocks,
                                          const int* doc_start, void* out, float* lse, int batch, int hq, int hkv,
                                          int nq, int nkv, int head_dim, int c, int rank, int causal, int zigzag,
                                          int round_begin, int round_end, int dtype, int out_dtype,
                                          void* stream) {
  if (doc_start != nullptr && causal == 0) return fail(RA_ERR_ARG, "a document mask needs causal=1");
  if (out_dtype != RA_BF16 && out_dtype != RA_F32) return fail(RA_ERR_ARG, "unknown out_dtype %d", out_dtype);
  return forward(q, k_blocks, v_blocks, doc_start, out, lse, batch, hq, hkv, nq, nkv, head_dim, c, rank, causal,
                 zigzag, round_begin, round_end, dtype, stream, true, out_dtype);
}

extern "C" int ra_merge(const void* out_a, const float* lse_a, const void* out_b, const float* lse_b, void* out,
                        float* lse, long long rows, int head_dim, int dtype, void* stream) {
  if (dtype != RA_BF16 && dtype != RA_F32) return fail(RA_ERR_ARG, "unknown dtype %d", dtype);
  if (rows < 0) return fail(RA_ERR_ARG, "rows=%lld must be >= 0", rows);
  if (head_dim < 8 || head_dim > 512 || head_dim % 8 != 0)
    return fail(RA_ERR_UNSUPPORTED, "merge needs head_dim a multiple of 8 in [8, 512] (got %d)", head_dim);
  if (rows > (LLONG_MAX >> 7)) return fail(RA_ERR_ARG, "rows=%lld too large", rows);
  if (rows == 0) return RA_OK;
  if (!out_a || !lse_a || !out_b || !lse_b || !out || !lse) return fail(RA_ERR_ARG, "NULL pointer");
  if (!aligned(out_a, 16) || !aligned(out_b, 16) || !aligned(out, 16))
    return fail(RA_ERR_ALIGN, "out_a, out_b and out must be 16-byte aligned");
  if (!aligned(lse_a, 4) || !aligned(lse_b, 4) || !aligned(lse, 4))
    return fail(RA_ERR_ALIGN, "lse arrays must be 4-byte aligned");
  hipError_t e = ra::launch_merge(out_a, lse_a, out_b, lse_b, out, lse, rows, head_dim, dtype,
                                  static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(RA_ERR_LAUNCH, "launch failed: %s", hipGetErrorString(e));
  return RA_OK;
}
