// attn_bwd.hip - backward kernels: preprocess, main (dK, dV and dQ contributions), dQ convert.
//
// The backward rebuilds P from the saved log-sum-exp instead of storing it, with the same
// mask unit as the forward ("Causal Mask and Ragged Sequence Layouts", sixth section:
// backward recomputation must rebuild the same logical mask), and sums the K/V gradients
// over each GQA group ("Attention Algorithm Error and Complexity Tests", third section).
// Per (query, key) pair, with c = scale * log2(e):
//   P   = exp2(c S - LSE log2 e)  (0 for disallowed pairs and out-of-range lanes)
//   dV += P^T dO          dP = dO V^T          dS = P (dP - D),  D = rowsum(dO * O)
//   dK += scale dS^T Q    dQ += scale dS K
//
// Main kernel: one workgroup = 4 waves = 128 keys of one (sequence, K/V head); wave w owns
// keys 32w..32w+31 and keeps their K, V (MFMA operands) and dK, dV (accumulators) in
// registers for the whole kernel, looping over every query head of the group and every
// 64-query tile that can see them. S = Q K^T and dP = dO V^T are computed with keys on the
// lanes (accumulator column = key), so P and dS are directly the right-hand operands of
// dV^T = dO^T P and dK^T = Q^T dS (left operands dO^T and Q^T come from LDS with transpose
// reads). dQ needs dS with queries on the lanes: dS goes through LDS, and the 4 waves split
// the 64 x head_dim dQ tile, each contracting over all 128 keys and adding its block into
// an fp32 dQ workspace with atomics.
#include "attn_device.hpp"
#include "attn_internal.h"

namespace attn {

constexpr int BWD_BN = 128;  // keys per workgroup
constexpr int BWD_BM = 64;   // queries per iteration

// Register-staged tile copy: global -> registers -> LDS (padded rows), 16 bytes per access.
// Rows at or beyond `valid_rows` are zero-filled and never read from memory.
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
      r[i] = row < valid_rows ? *reinterpret_cast<const i32x4*>(base + row * row_stride_bytes + c * 16)
                              : i32x4{0, 0, 0, 0};
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

struct BwdParams {
  const __bf16* q;
  const __bf16* k;
  const __bf16* v;
  const __bf16* dout;
  const int32_t* cu_q;
  const int32_t* cu_k;
  int num_seqs, total_q, hq, hkv, group;
  float c;       // scale * log2(e), signed
  float scale;
  int mode, window;
  const float* lse2;   // [hq, total_q] LSE * log2(e); +inf for rows with no allowed key
  const float* dvec;   // [hq, total_q] rowsum(dO * O)
  float* dq_acc;       // [total_q, hq, D] fp32
  __bf16* dk;
  __bf16* dv;
  int nslots, nlogical;
};

// Query positions [lo, hi) that can see any key position in [k0, k1) (k1 > k0).
__device__ __forceinline__ void visible_queries(int k0, int k1, const SeqGeom& g, int mode,
                                                int window, int& lo, int& hi) {
  if (mode == MASK_NONE) {
    lo = 0;
    hi = g.len_q;
    return;
  }
  lo = max(0, k0 - g.off);  // key k visible from q iff q >= k - off (and q < k - off + W)
  hi = window > 0 ? min(g.len_q, k1 - 1 - g.off + window) : g.len_q;
  if (hi < lo) hi = lo;
}

// ---------------------------------------------------------------------------------------
// Preprocess: D = rowsum(dO * O) in fp32 from the stored output, LSE -> log2 units with
// empty rows mapped to +inf (so every recomputed P of such a row is exactly 0), and the
// fp32 dQ accumulator cleared. One wave per (query token, query head).
// ---------------------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(const T* __restrict__ out,
                                                      const T* __restrict__ dout,
                                                      const float* __restrict__ lse, int total_q,
                                                      int hq, float* __restrict__ dvec,
                                                      float* __restrict__ lse2,
                                                      float* __restrict__ dq_acc) {
  const int lane = threadIdx.x & 63;
  const long item = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (item >= (long)total_q * hq) return;
  const int t = (int)(item / hq), h = (int)(item - (long)t * hq);
  constexpr int PER = D / 64;
  const size_t base = ((size_t)t * hq + h) * D + lane * PER;
  float acc = 0.0f;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    acc += (float)dout[base + i] * (float)out[base + i];
    dq_acc[base + i] = 0.0f;
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off);
  if (lane == 0) {
    const size_t li = (size_t)h * total_q + t;
    dvec[li] = acc;
    const float l = lse[li];
    lse2[li] = (l == neg_inf()) ? __builtin_inff() : l * LOG2E;
  }
}

template <typename T, int D>
__global__ __launch_bounds__(256) void bwd_dq_convert_kernel(const float* __restrict__ dq_acc,
                                                             T* __restrict__ dq, long n) {
  const long i = ((long)blockIdx.x * blockDim.x + threadIdx.x) * 4;
  if (i >= n) return;
  const f32x4 x = *reinterpret_cast<const f32x4*>(dq_acc + i);
  Mma<T, D>::store4(dq + i, x[0], x[1], x[2], x[3]);
}

// ---------------------------------------------------------------------------------------
// Main backward kernel (bf16).
// ---------------------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256, 1) void bwd_main_kernel(BwdParams p) {
  typedef Mma<__bf16, D> M;
  constexpr int PITCH = D * 2 + 16;               // Q, dO, K rows: D bf16 + 16 bytes
  constexpr int SPITCH = BWD_BN * 2 + 16;         // dS rows: 128 keys bf16 + 16 bytes
  constexpr int NDB = D / 32;
  constexpr int QREGS = D / 16;
  __shared__ __attribute__((aligned(16))) char ks[BWD_BN * PITCH];
  __shared__ __attribute__((aligned(16))) char qs[BWD_BM * PITCH];
  __shared__ __attribute__((aligned(16))) char dos[BWD_BM * PITCH];
  __shared__ __attribute__((aligned(16))) char dss[BWD_BM * SPITCH];
  __shared__ float lse2s[BWD_BM];
  __shared__ float dvs[BWD_BM];

  const int tid = threadIdx.x, lane = tid & 63, wave = uniform(tid >> 6);
  const int hg = lane >> 5;
  const int w = xcd_logical_block(blockIdx.x, p.nlogical);
  if (w < 0) return;
  const int kvh = w / p.nslots, slot = w - kvh * p.nslots;
  const int s = seq_of_slot<BWD_BN>(p.cu_k, p.num_seqs, slot);
  const SeqGeom g = load_geom(p.cu_q, p.cu_k, s, p.mode);
  const int ntiles = (g.len_k + BWD_BN - 1) / BWD_BN;
  const int kt = slot - (g.k_start / BWD_BN + s);
  if (kt >= ntiles) return;
  const int k0 = kt * BWD_BN, k1 = min(k0 + BWD_BN, g.len_k);
  const int kw0 = k0 + 32 * wave;                 // this wave's first key position
  const int kj = kw0 + (lane & 31);               // this lane's key position
  const bool kvalid = kj < k1;

  const size_t krs = (size_t)p.hkv * D;           // K/V row stride (elements)
  const __bf16* kbase = p.k + ((size_t)g.k_start * p.hkv + kvh) * D;
  const __bf16* vbase = p.v + ((size_t)g.k_start * p.hkv + kvh) * D;

  // K^T / V^T operands: lane (key j, half g) holds row j, head-dim 16 s + 8 g + 0..7.
  bf16x8 kr[QREGS], vr[QREGS];
#pragma unroll
  for (int st = 0; st < QREGS; ++st) {
    const size_t off = (size_t)kj * krs + 16 * st + 8 * hg;
    const i32x4 z = {0, 0, 0, 0};
    kr[st] = __builtin_bit_cast(bf16x8, kvalid ? *reinterpret_cast<const i32x4*>(kbase + off) : z);
    vr[st] = __builtin_bit_cast(bf16x8, kvalid ? *reinterpret_cast<const i32x4*>(vbase + off) : z);
  }
  // K tile in LDS (rows beyond the sequence are zero) for the dQ contraction.
  {
    typedef RowStager<D * 2, BWD_BN, 256> Stager;
    Stager st;
    st.load(reinterpret_cast<const char*>(kbase + (size_t)k0 * krs), krs * 2, k1 - k0, tid);
    st.store(ks, PITCH, tid);
  }

  f32x16 dka[NDB], dva[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    dka[db] = f32x16{};
    dva[db] = f32x16{};
  }

  int qlo, qhi;
  visible_queries(k0, k1, g, p.mode, p.window, qlo, qhi);
  const int qstart = (qlo / BWD_BM) * BWD_BM;
  const int nqt = qhi > qlo ? (qhi - qstart + BWD_BM - 1) / BWD_BM : 0;
  const int niter = nqt * p.group;

  typedef RowStager<D * 2, BWD_BM, 256> QStager;
  QStager sq, sdo;
  const size_t qrs = (size_t)p.hq * D;
  auto tile_ptrs = [&](int it, int& h, int& q0) {
    h = kvh * p.group + it / nqt;
    q0 = qstart + (it % nqt) * BWD_BM;
  };
  if (niter > 0) {
    int h, q0;
    tile_ptrs(0, h, q0);
    const size_t off = ((size_t)(g.q_start + q0) * p.hq + h) * D;
    sq.load(reinterpret_cast<const char*>(p.q + off), qrs * 2, g.len_q - q0, tid);
    sdo.load(reinterpret_cast<const char*>(p.dout + off), qrs * 2, g.len_q - q0, tid);
  }

  const int a16 = lane & 15, hh = (lane >> 4) & 1;
  for (int it = 0; it < niter; ++it) {
    int h, q0;
    tile_ptrs(it, h, q0);
    const int qend = min(q0 + BWD_BM, g.len_q);
    // Stage this tile's Q, dO, LSE and D (rows beyond the sequence: zeros / +inf LSE).
    sq.store(qs, PITCH, tid);
    sdo.store(dos, PITCH, tid);
    if (tid < BWD_BM) {
      const int pq = q0 + tid;
      const size_t li = (size_t)h * p.total_q + g.q_start + pq;
      lse2s[tid] = pq < g.len_q ? p.lse2[li] : __builtin_inff();
      dvs[tid] = pq < g.len_q ? p.dvec[li] : 0.0f;
    }
    __syncthreads();
    if (it + 1 < niter) {
      int hn, qn;
      tile_ptrs(it + 1, hn, qn);
      const size_t off = ((size_t)(g.q_start + qn) * p.hq + hn) * D;
      sq.load(reinterpret_cast<const char*>(p.q + off), qrs * 2, g.len_q - qn, tid);
      sdo.load(reinterpret_cast<const char*>(p.dout + off), qrs * 2, g.len_q - qn, tid);
    }

#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const int qa = q0 + 32 * qb, qz = min(qa + 32, qend);
      const int cls = block_class(qa, qz, kw0, kw0 + 32, g, p.mode, p.window);
      bf16x8 pb[2], dsb[2];
      if (cls != 0) {
        // S and dP with keys on the lanes: A = Q / dO rows from LDS, B = K / V registers.
        f32x16 sacc = f32x16{}, dpacc = f32x16{};
        const char* qp = qs + (32 * qb + (lane & 31)) * PITCH + hg * 16;
        const char* dp = dos + (32 * qb + (lane & 31)) * PITCH + hg * 16;
#pragma unroll
        for (int st = 0; st < QREGS; ++st) {
          sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              *reinterpret_cast<const bf16x8*>(qp + st * 32), kr[st], sacc, 0, 0, 0);
          dpacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              *reinterpret_cast<const bf16x8*>(dp + st * 32), vr[st], dpacc, 0, 0, 0);
        }
        // P and dS; register r holds query row 32 qb + key_of_reg(r, g).
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = 32 * qb + key_of_reg(r, hg);
          const bool ok = (cls == 2) | pair_allowed(q0 + row, kj, g, p.mode, p.window);
          const float pv = ok ? fast_exp2(fmaf(sacc[r], p.c, -lse2s[row])) : 0.0f;
          sacc[r] = pv;
          dpacc[r] = pv * (dpacc[r] - dvs[row]);
        }
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          pb[0][t] = (__bf16)sacc[t];
          pb[1][t] = (__bf16)sacc[8 + t];
          dsb[0][t] = (__bf16)dpacc[t];
          dsb[1][t] = (__bf16)dpacc[8 + t];
        }
        // dV^T += dO^T P and dK^T += Q^T dS over this block's 32 queries (two 16-query
        // steps; transpose reads give rows 16 s + 8 j + 4 g + 0..3 of column l % 32).
        const char* dob = dos + (32 * qb + 4 * hg + (a16 >> 2)) * PITCH + (16 * hh + 4 * (a16 & 3)) * 2;
        const char* qbp = qs + (32 * qb + 4 * hg + (a16 >> 2)) * PITCH + (16 * hh + 4 * (a16 & 3)) * 2;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int st = 0; st < 2; ++st) {
            const int o = 16 * st * PITCH + db * 64;
            const i16x4 d0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(dob + o));
            const i16x4 d1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(dob + o + 8 * PITCH));
            const i16x4 q0r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(qbp + o));
            const i16x4 q1r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(qbp + o + 8 * PITCH));
            const i32x4 da = {__builtin_bit_cast(i32x2, d0)[0], __builtin_bit_cast(i32x2, d0)[1],
                              __builtin_bit_cast(i32x2, d1)[0], __builtin_bit_cast(i32x2, d1)[1]};
            const i32x4 qa4 = {__builtin_bit_cast(i32x2, q0r)[0], __builtin_bit_cast(i32x2, q0r)[1],
                               __builtin_bit_cast(i32x2, q1r)[0], __builtin_bit_cast(i32x2, q1r)[1]};
            dva[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, da), pb[st],
                                                              dva[db], 0, 0, 0);
            dka[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, qa4), dsb[st],
                                                              dka[db], 0, 0, 0);
          }
      } else {
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          dsb[0][t] = (__bf16)0.0f;
          dsb[1][t] = (__bf16)0.0f;
        }
      }
      // dS -> LDS as [query row][key] (bf16) for the dQ contraction.
      __bf16* dsrow = reinterpret_cast<__bf16*>(dss + 64 * wave + (lane & 31) * 2);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = 32 * qb + key_of_reg(r, hg);
        *reinterpret_cast<__bf16*>(reinterpret_cast<char*>(dsrow) + row * SPITCH) =
            dsb[r >> 3][r & 7];
      }
    }
    __syncthreads();

    // dQ tile (64 queries x D): wave w takes query block w / 2 and half of the head-dim
    // blocks; A = dS rows (8 consecutive keys per lane), B = K via transpose reads.
    {
      const int qb = wave >> 1;
      constexpr int DPW = NDB / 2;   // head-dim blocks per wave
      const char* ap = dss + (32 * qb + (lane & 31)) * SPITCH + hg * 16;
#pragma unroll
      for (int i = 0; i < DPW; ++i) {
        const int db = (wave & 1) * DPW + i;
        f32x16 acc = f32x16{};
        const char* bp = ks + (8 * hg + (a16 >> 2)) * PITCH + (db * 32 + 16 * hh + 4 * (a16 & 3)) * 2;
#pragma unroll
        for (int st = 0; st < BWD_BN / 16; ++st) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(ap + st * 32);
          const i16x4 b0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(bp + 16 * st * PITCH));
          const i16x4 b1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(bp + (16 * st + 4) * PITCH));
          const i32x4 bb = {__builtin_bit_cast(i32x2, b0)[0], __builtin_bit_cast(i32x2, b0)[1],
                            __builtin_bit_cast(i32x2, b1)[0], __builtin_bit_cast(i32x2, b1)[1]};
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, __builtin_bit_cast(bf16x8, bb), acc, 0, 0, 0);
        }
        // Accumulator: column = head-dim db*32 + l%32, row = query 32 qb + key_of_reg(r, g).
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int pq = q0 + 32 * qb + key_of_reg(r, hg);
          if (pq < qend) {
            float* dst = p.dq_acc + ((size_t)(g.q_start + pq) * p.hq + h) * D + db * 32 + (lane & 31);
            atomicAdd(dst, acc[r] * p.scale);
          }
        }
      }
    }
    __syncthreads();
  }

  // dK = scale * sum dS^T Q, dV = sum P^T dO; accumulator column = key, rows = head dim.
  if (kvalid) {
    __bf16* dkrow = p.dk + ((size_t)(g.k_start + kj) * p.hkv + kvh) * D;
    __bf16* dvrow = p.dv + ((size_t)(g.k_start + kj) * p.hkv + kvh) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int d = db * 32 + 8 * a + 4 * hg;
        M::store4(dkrow + d, dka[db][4 * a] * p.scale, dka[db][4 * a + 1] * p.scale,
                  dka[db][4 * a + 2] * p.scale, dka[db][4 * a + 3] * p.scale);
        M::store4(dvrow + d, dva[db][4 * a], dva[db][4 * a + 1], dva[db][4 * a + 2], dva[db][4 * a + 3]);
      }
  }
}

// ---------------------------------------------------------------------------------------
// Launch
// ---------------------------------------------------------------------------------------
size_t bwd_workspace_bytes(int total_q, int hq, int d) {
  const size_t dq = (size_t)total_q * hq * d * sizeof(float);
  const size_t vec = (size_t)total_q * hq * sizeof(float);
  return ((dq + 255) / 256) * 256 + 2 * (((vec + 255) / 256) * 256);
}

template <int D>
static hipError_t bwd_typed(const BwdArgs& a, void* ws, hipStream_t st) {
  const FwdArgs& f = a.f;
  const size_t dqb = (((size_t)f.total_q * f.hq * D * sizeof(float) + 255) / 256) * 256;
  const size_t vecb = (((size_t)f.total_q * f.hq * sizeof(float) + 255) / 256) * 256;
  float* dq_acc = static_cast<float*>(ws);
  float* dvec = reinterpret_cast<float*>(static_cast<char*>(ws) + dqb);
  float* lse2 = reinterpret_cast<float*>(static_cast<char*>(ws) + dqb + vecb);
  const long items = (long)f.total_q * f.hq;
  if (items > 0) {
    hipLaunchKernelGGL((bwd_pre_kernel<__bf16, D>), dim3((unsigned)((items + 3) / 4)), dim3(256), 0, st,
                       static_cast<const __bf16*>(a.out), static_cast<const __bf16*>(a.dout), a.lse,
                       f.total_q, f.hq, dvec, lse2, dq_acc);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  BwdParams p{};
  p.q = static_cast<const __bf16*>(f.q);
  p.k = static_cast<const __bf16*>(f.k);
  p.v = static_cast<const __bf16*>(f.v);
  p.dout = static_cast<const __bf16*>(a.dout);
  p.cu_q = f.cu_q;
  p.cu_k = f.cu_k;
  p.num_seqs = f.num_seqs;
  p.total_q = f.total_q;
  p.hq = f.hq;
  p.hkv = f.hkv;
  p.group = f.hq / f.hkv;
  p.c = (float)((double)f.scale * 1.4426950408889634);
  p.scale = f.scale;
  p.mode = f.mode;
  p.window = f.window;
  p.lse2 = lse2;
  p.dvec = dvec;
  p.dq_acc = dq_acc;
  p.dk = static_cast<__bf16*>(a.dk);
  p.dv = static_cast<__bf16*>(a.dv);
  p.nslots = f.total_k / BWD_BN + f.num_seqs;
  p.nlogical = p.nslots * f.hkv;
  if (f.total_k > 0) {
    const int grid = ((p.nlogical + 7) / 8) * 8;
    hipLaunchKernelGGL((bwd_main_kernel<D>), dim3(grid), dim3(256), 0, st, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const long n = (long)f.total_q * f.hq * D;
  if (n > 0) {
    hipLaunchKernelGGL((bwd_dq_convert_kernel<__bf16, D>), dim3((unsigned)((n / 4 + 255) / 256)), dim3(256),
                       0, st, dq_acc, static_cast<__bf16*>(a.dq), n);
  }
  return hipGetLastError();
}

hipError_t launch_bwd(const BwdArgs& a, void* ws, hipStream_t st) {
  if (a.f.dtype != 0) return hipErrorNotSupported;
  return a.f.d == 64 ? bwd_typed<64>(a, ws, st) : bwd_typed<128>(a, ws, st);
}

}  // namespace attn
