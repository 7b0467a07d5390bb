// attn_device.hpp - device building blocks of the exact tiled attention kernels (gfx950).
//
// Everything here is CDNA4-specific: 64-lane wavefronts, the 32x32 MFMA accumulator
// layout, LDS transpose reads, and XCD round-robin workgroup dispatch.
//
// MFMA 32x32 accumulator layout (measured on gfx950 for v_mfma_f32_32x32x16_bf16 and
// v_mfma_f32_32x32x2_f32): lane l, register r holds C[row][col] with
//     col = l % 32,   row = 8 * (r / 4) + 4 * (l / 32) + (r % 4).
// Operands of 32x32x16 bf16: lane l holds A[l % 32][8 * (l / 32) + t] and
// B[8 * (l / 32) + t][l % 32] for t = 0..7. Operands of 32x32x2 f32: lane l holds
// A[l % 32][l / 32] and B[l / 32][l % 32].
//
// The forward computes S^T = K Q^T (rows = keys, columns = queries), so after the QK^T
// contraction every lane owns ONE query (column l % 32) and 16 of the 32 keys of a block:
// the softmax row statistics are per-lane values plus one exchange with lane l ^ 32, and
// the P^T operand of the following O^T = V^T P^T contraction is already in registers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) short i16x4;
typedef __attribute__((ext_vector_type(4))) int i32x4;
typedef __attribute__((ext_vector_type(2))) int i32x2;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int WAVE = 64;
constexpr int LDS_BYTES = 160 * 1024;  // per workgroup on gfx950
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;
constexpr int MASK_NONE = 0;
constexpr int MASK_TOP_LEFT = 1;
constexpr int MASK_BOTTOM_RIGHT = 2;

__device__ __forceinline__ float neg_inf() { return -__builtin_inff(); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Value of the same register in lane l ^ 32 (the other half of the wave).
__device__ __forceinline__ float swap_halves(float x) {
  return __shfl_xor(x, 32);
}

// ---------------------------------------------------------------------------------------
// Mask unit. Sequence geometry comes from cu_seqlens; positions are always in-sequence
// (0-based), never packed offsets. `off` is the alignment shift of the causal diagonal:
// 0 for top-left, len_k - len_q for bottom-right.
// ---------------------------------------------------------------------------------------
struct SeqGeom {
  int q_start, k_start;  // packed offsets of the sequence's first query / key token
  int len_q, len_k;
  int off;
};

__device__ __forceinline__ SeqGeom load_geom(const int32_t* cu_q, const int32_t* cu_k, int s,
                                             int mode) {
  SeqGeom g;
  g.q_start = cu_q[s];
  g.k_start = cu_k[s];
  g.len_q = cu_q[s + 1] - g.q_start;
  g.len_k = cu_k[s + 1] - g.k_start;
  g.off = (mode == MASK_BOTTOM_RIGHT) ? g.len_k - g.len_q : 0;
  return g;
}

// Is key position pk visible from query position pq? Out-of-range key lanes (pk >= len_k)
// are excluded like any disallowed pair. Branch-free on purpose: callers turn the result
// into a select, never into a divergent conditional store.
__device__ __forceinline__ bool pair_allowed(int pq, int pk, const SeqGeom& g, int mode,
                                             int window) {
  const int end = pq + g.off;
  const bool causal_ok = (pk <= end) & ((window <= 0) | (pk > end - window));
  return (pk < g.len_k) & ((mode == MASK_NONE) | causal_ok);
}

// Key positions [lo, hi) that any query position in [p0, p1) may see (p1 > p0).
__device__ __forceinline__ void visible_keys(int p0, int p1, const SeqGeom& g, int mode,
                                             int window, int& lo, int& hi) {
  if (mode == MASK_NONE) {
    lo = 0;
    hi = g.len_k;
    return;
  }
  hi = min(g.len_k, p1 + g.off);  // largest visible key is (p1 - 1) + off
  lo = window > 0 ? max(0, p0 + g.off - window + 1) : 0;
  if (hi < lo) hi = lo;
}

// Classification of a (query positions [p0,p1)) x (key positions [k0,k1)) block:
// 0 = no pair allowed, 1 = some pairs (per-lane test needed), 2 = every pair allowed.
__device__ __forceinline__ int block_class(int p0, int p1, int k0, int k1, const SeqGeom& g,
                                           int mode, int window) {
  if (p1 <= p0 || k0 >= g.len_k || k1 <= k0) return 0;
  if (mode != MASK_NONE) {
    if (k0 > p1 - 1 + g.off) return 0;                              // all keys in the future
    if (window > 0 && k1 - 1 <= p0 + g.off - window) return 0;      // all keys out of window
  }
  if (k1 > g.len_k) return 1;
  if (mode == MASK_NONE) return 2;
  if (k1 - 1 > p0 + g.off) return 1;
  if (window > 0 && k0 <= p1 - 1 + g.off - window) return 1;
  return 2;
}

// Sequence owning packed token t: largest s with cu[s] <= t, skipping empty sequences.
__device__ __forceinline__ int seq_of_token(const int32_t* cu, int num_seqs, int t) {
  int lo = 0, hi = num_seqs - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (cu[mid] <= t) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// ---------------------------------------------------------------------------------------
// Varlen tile scheduler. Query tiles of BM rows start at each sequence's first token.
// Sequence s owns the slot range starting at floor(cu_q[s] / BM) + s; it uses its first
// ceil(len_q / BM) slots and the rest exit at once. Because floor(c / BM) + ceil(L / BM)
// <= floor((c + L) / BM) + 1, slot ranges never overlap, and floor(total_q / BM) +
// num_seqs slots cover every tile. The owner of a slot is found by binary search on
// cu_q, so the host never reads cu_seqlens and no prepass is needed.
// ---------------------------------------------------------------------------------------
template <int BM>
__device__ __forceinline__ int seq_of_slot(const int32_t* cu_q, int num_seqs, int slot) {
  int lo = 0, hi = num_seqs - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (cu_q[mid] / BM + mid <= slot) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Workgroups are handed to the 8 XCDs round-robin (block b runs on XCD b % 8). This maps
// the hardware block id to a logical work index so that consecutive logical items (the
// query tiles of one head and sequence, which read the same K/V) run on the same XCD and
// share its L2. Returns -1 for padding blocks.
__device__ __forceinline__ int xcd_logical_block(int b, int nlogical) {
  const int per = (nlogical + 7) >> 3;
  const int w = (b & 7) * per + (b >> 3);
  return w < nlogical ? w : -1;
}

// ---------------------------------------------------------------------------------------
// K/V staging: global -> registers -> LDS, 16 bytes per access. Rows at or beyond
// `valid_rows` are zero-filled and never read from memory (no access past the sequence's
// last key, so nothing past the end of the tensor either).
// ---------------------------------------------------------------------------------------
template <int ROW_BYTES, int ROWS, int NTHREADS>
struct RowStager {
  static constexpr int CHUNKS = ROW_BYTES / 16;
  static constexpr int TOTAL = ROWS * CHUNKS;
  static_assert(TOTAL % NTHREADS == 0, "tile must split evenly over the threads");
  static constexpr int PER_THREAD = TOTAL / NTHREADS;
  i32x4 r[PER_THREAD];

  __device__ __forceinline__ void load(const char* base, size_t row_stride_bytes, int valid_rows,
                                       int tid) {
#pragma unroll
    for (int i = 0; i < PER_THREAD; ++i) {
      const int idx = i * NTHREADS + tid;
      const int row = idx / CHUNKS, c = idx % CHUNKS;
      if (row < valid_rows) {
        r[i] = *reinterpret_cast<const i32x4*>(base + row * row_stride_bytes + c * 16);
      } else {
        r[i] = i32x4{0, 0, 0, 0};
      }
    }
  }
  __device__ __forceinline__ void store(char* lds, int pitch, int tid) const {
#pragma unroll
    for (int i = 0; i < PER_THREAD; ++i) {
      const int idx = i * NTHREADS + tid;
      const int row = idx / CHUNKS, c = idx % CHUNKS;
      *reinterpret_cast<i32x4*>(lds + row * pitch + c * 16) = r[i];
    }
  }
};

// ---------------------------------------------------------------------------------------
// Element-type specific contractions. Key k of a 32-key block sits in register r of lane
// half g = l / 32 with k = 8 * (r / 4) + 4 * g + (r % 4) (the accumulator layout above).
// ---------------------------------------------------------------------------------------
__device__ __forceinline__ int key_of_reg(int r, int g) { return 8 * (r >> 2) + 4 * g + (r & 3); }

template <typename T, int D>
struct Mma;

// bf16: v_mfma_f32_32x32x16_bf16 for both contractions; V^T operands via ds_read_b64_tr_b16.
template <int D>
struct Mma<__bf16, D> {
  static constexpr int PITCH = D * 2 + 16;  // LDS row pitch (bytes): +16 spreads rows over banks
  static constexpr int QREGS = D / 16;
  typedef bf16x8 QOperand;

  // Q^T operand of S^T = K Q^T: lane (q = l % 32, g = l / 32) holds q[16 s + 8 g + 0..7].
  // `neg` flips the sign bit (exact) so a negative scale becomes a positive one.
  __device__ static void load_q(QOperand (&qr)[QREGS], const __bf16* qrow, bool valid, bool neg,
                                int lane) {
    const int g = lane >> 5;
#pragma unroll
    for (int s = 0; s < QREGS; ++s) {
      i32x4 x = valid ? *reinterpret_cast<const i32x4*>(qrow + 16 * s + 8 * g) : i32x4{0, 0, 0, 0};
      if (neg) x ^= i32x4{(int)0x80008000, (int)0x80008000, (int)0x80008000, (int)0x80008000};
      qr[s] = __builtin_bit_cast(bf16x8, x);
    }
  }

  // acc += K_block Q^T over the full head dimension; kl points at LDS row 0 of the block.
  __device__ static void qk(f32x16& acc, const char* kl, const QOperand (&qr)[QREGS], int lane) {
    const char* p = kl + (lane & 31) * PITCH + (lane >> 5) * 16;
#pragma unroll
    for (int s = 0; s < QREGS; ++s) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(p + s * 32);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qr[s], acc, 0, 0, 0);
    }
  }

  // o[db] += V_block^T P^T for the 32 keys of one block; p holds P^T in accumulator layout.
  // K-slot t = 4 j + u of step s carries key 16 s + 8 j + 4 g + u, which is register
  // 8 s + t of p, and is what the two transpose reads (rows +0 and +8) return.
  __device__ static void pv(f32x16 (&o)[D / 32], const f32x16& p, const char* vl, int lane) {
    bf16x8 b[2];
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      b[0][t] = (__bf16)p[t];
      b[1][t] = (__bf16)p[8 + t];
    }
    const int a16 = lane & 15, hh = (lane >> 4) & 1, g = lane >> 5;
    const char* base = vl + (4 * g + (a16 >> 2)) * PITCH + (16 * hh + 4 * (a16 & 3)) * 2;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const char* p0 = base + 16 * s * PITCH + db * 64;
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p0));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p0 + 8 * PITCH));
        const i32x4 cat = {__builtin_bit_cast(i32x2, lo)[0], __builtin_bit_cast(i32x2, lo)[1],
                           __builtin_bit_cast(i32x2, hi)[0], __builtin_bit_cast(i32x2, hi)[1]};
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, cat), b[s],
                                                        o[db], 0, 0, 0);
      }
    }
  }

  // Output element type conversion: four consecutive head-dim values -> 8 bytes.
  __device__ static void store4(__bf16* dst, float a, float b, float c, float d) {
    typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
    bf16x4 v = {(__bf16)a, (__bf16)b, (__bf16)c, (__bf16)d};
    *reinterpret_cast<bf16x4*>(dst) = v;
  }
};

// fp32: v_mfma_f32_32x32x2_f32 (exact products, fp32 accumulation).
template <int D>
struct Mma<float, D> {
  static constexpr int PITCH = D * 4 + 16;
  static constexpr int QREGS = D / 2;
  typedef float QOperand;

  __device__ static void load_q(QOperand (&qr)[QREGS], const float* qrow, bool valid, bool neg,
                                int lane) {
    const int g = lane >> 5;
#pragma unroll
    for (int s = 0; s < QREGS; ++s) {
      const float x = valid ? qrow[2 * s + g] : 0.0f;
      qr[s] = neg ? -x : x;
    }
  }

  __device__ static void qk(f32x16& acc, const char* kl, const QOperand (&qr)[QREGS], int lane) {
    const float* p = reinterpret_cast<const float*>(kl + (lane & 31) * PITCH) + (lane >> 5);
#pragma unroll
    for (int s = 0; s < QREGS; ++s) {
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(p[2 * s], qr[s], acc, 0, 0, 0);
    }
  }

  // Step r contracts the two keys held in register r by the two lane halves.
  __device__ static void pv(f32x16 (&o)[D / 32], const f32x16& p, const char* vl, int lane) {
    const int i = lane & 31, g = lane >> 5;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float a =
            *reinterpret_cast<const float*>(vl + key_of_reg(r, g) * PITCH + (db * 32 + i) * 4);
        o[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, p[r], o[db], 0, 0, 0);
      }
    }
  }

  __device__ static void store4(float* dst, float a, float b, float c, float d) {
    *reinterpret_cast<f32x4*>(dst) = f32x4{a, b, c, d};
  }
};

}  // namespace attn
