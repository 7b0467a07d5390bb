// attn_internal.h - launch interface between the C ABI layer and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace attn {

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* cu_q;
  const int32_t* cu_k;
  int num_seqs, total_q, total_k, max_q, max_k;
  int hq, hkv, d, dtype;
  float scale;
  int mode, window;
  void* out;
  float* lse;
  // dropout on the attention weights: thr = round(256 p) in 1..255 (0 = none), scale =
  // 1 / (1 - thr / 256), 64-bit seed of the counter-based generator
  uint32_t drop_thr = 0;
  float drop_scale = 1.0f;
  uint64_t seed = 0;
  // bf16 forward through attn_fwd_dropout only (may be null): O - round_bf16(O) per output
  // element, in bf16
  void* out_res = nullptr;
};

struct BwdArgs {
  FwdArgs f;          // q, k, v, cu, sizes, scale, mask (out/lse: forward outputs)
  const void* out;
  const void* out_res = nullptr;  // bf16 (attn_bwd_dropout only): the forward's residual
  const float* lse;
  const void* dout;
  void* dq;
  void* dk;
  void* dv;
};

// Forward prefill tile shape (query rows per workgroup, keys per LDS stage).
constexpr int FWD_BM = 128;
constexpr int FWD_BN = 64;
// Split-K decode: keys per LDS stage (32 per wave) and the largest query-row count per
// K/V head it supports (two 32-row blocks per wave).
constexpr int SPLITK_STAGE = 128;
constexpr int SPLITK_MAX_ROWS = 64;

// True when every sequence has exactly max_q queries and max_k keys; the prefill then
// orders its tiles heaviest first across all (sequence, head) pairs.
bool equal_lengths(const FwdArgs& a);
int fwd_prefill_grid(const FwdArgs& a);
// Other batches sort their tiles by cost first (a small kernel writing the order into the
// workspace: one int32 per slot).
size_t fwd_prefill_workspace_bytes(const FwdArgs& a);
hipError_t launch_fwd_prefill(const FwdArgs& a, void* workspace, hipStream_t stream);
// keep[i * nk + j] (uint8) of dropout element (q0 + i, k0 + j) of sequence s, query head h.
hipError_t launch_dropout_probe(uint64_t seed, uint32_t thr, int s, int h, int q0, int nq, int k0,
                                int nk, uint8_t* keep, hipStream_t stream);

// Partials per key chunk of the split-K path (the waves of a workgroup merge theirs).
int splitk_partials_per_chunk(int rows);
size_t splitk_workspace_bytes(int nsplit_eff, int total_q, int hq, int d);
hipError_t launch_fwd_splitk(const FwdArgs& a, int blocks_per_kvh, int chunk, void* workspace,
                             hipStream_t stream);

// Well-formedness of cu_seqlens (include/attn.h, attn_check_seqlens): one workgroup ORs the
// attn_seqlens_error bits of every sequence and writes the word.
hipError_t launch_check_seqlens(const int32_t* cu_q, const int32_t* cu_k, int num_seqs,
                                int total_q, int total_k, int max_q, int max_k, int32_t* word,
                                hipStream_t stream);

// Mask probes (one kernel unit's exclusion decisions replayed into a uint8 [nq, nk] array;
// include/attn.h, attn_mask_probe_ex). unit: 0 bf16 prefill, 1 generic prefill (fp32,
// dropout), 2 split-K decode (plan nsb / chunk / nrb, query head `head`), 3 backward dK/dV
// kernel, 4 backward dQ kernel, 5 and 6 the same two in fp32.
struct ProbeArgs {
  const int32_t* cu_q;
  const int32_t* cu_k;
  int num_seqs, mode, window, unit;
  int group, head, nsb, chunk, nrb;  // split-K only
  int q0, nq, k0, nk;
};
hipError_t launch_probe_zero(uint8_t* bits, long n, hipStream_t stream);
hipError_t launch_mask_probe_fwd(const ProbeArgs& a, uint8_t* bits, hipStream_t stream);
hipError_t launch_mask_probe_bwd(const ProbeArgs& a, uint8_t* bits, hipStream_t stream);

// Backward tile shape and workspace.
size_t bwd_workspace_bytes(int total_q, int hq, int d);
hipError_t launch_bwd(const BwdArgs& a, void* workspace, hipStream_t stream);

}  // namespace attn
