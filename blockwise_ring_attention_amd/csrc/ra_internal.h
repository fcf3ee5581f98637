// Internal interface between the host C ABI (ra_host.cpp) and the device code.
#pragma once

#include <hip/hip_runtime.h>

namespace ra {

// Everything a forward launch needs, computed and checked on the host.
struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* out;
  float* lse;           // may be null
  const int* doc;       // document starts by global position (causal document mask), or null
  int acc;              // 1: fold the result into the running (out, lse) in memory
  int out_f32;          // 1: out is fp32 (bf16 inputs, accumulate mode), else the input type
  int B, hq, hkv, nq, nkv, d;
  int c, rank, causal, zigzag, t0, t1;
  // Work decomposition (see plan_forward in ra_host.cpp).
  int G;                // hq / hkv: query heads per KV head
  int hpw;              // query heads packed into one workgroup (divides G)
  int hsets;            // G / hpw
  int prow;             // query rows (positions) per workgroup tile
  int nhalves;          // 2 when causal zigzag (tiles never straddle chunks), else 1
  int rows_half;        // nq / nhalves
  int tiles_half;       // ceil(rows_half / prow)
  int qtiles;           // nhalves * tiles_half
  int streams;          // B * hkv * hsets: independent (batch, KV head, head set) units
  int xcd_map;          // 1: (B * hkv) % 8 == 0, pin each KV head to one XCD
  float scale_log2;     // log2(e) / sqrt(d)
};

// Column blocks (of 32 query rows each) per workgroup, per kernel family.
constexpr int kBf16ColBlocks = 8;   // 8 waves x 1 column block
constexpr int kF32ColBlocks = 4;    // 4 waves x 1 column block

hipError_t launch_forward_bf16(const FwdArgs& a, int grid, hipStream_t stream);
hipError_t launch_forward_f32(const FwdArgs& a, int grid, hipStream_t stream);
hipError_t launch_merge(const void* oa, const float* la, const void* ob, const float* lb, void* out,
                        float* lse, long long rows, int d, int dtype, hipStream_t stream);

}  // namespace ra
