// attn_bwd.hip - backward kernels: dQ (query-major; for bf16 it also forms D and the LSE in
// base 2 and runs first), dK/dV (key-major), the preprocess used by fp32 and by dropout
// without the forward's output residual, and the fp32 kernels.
//
// The backward rebuilds P from the saved log-sum-exp instead of storing it, deciding which
// pairs count with the forward's own interval rules, so that its mask is the forward's
// ("Causal Mask and Ragged Sequence Layouts", sixth section), and sums the K/V gradients
// over each GQA group ("Attention Algorithm Error and Complexity Tests", third section).
// Per (query, key) pair, with c = scale * log2(e):
//   P   = exp2(c S - LSE log2 e)  (0 for disallowed pairs and out-of-range lanes)
//   dV += P^T dO          dP = dO V^T          dS = P (dP - D),  D = rowsum(dO * O)
//   dK += scale dS^T Q    dQ += scale dS K
//
// dK/dV kernel: one workgroup = 8 waves = 128 keys of one (sequence, K/V head), looping
// over every query head of the group and every 64-query tile that can see those keys (see
// bwd_main_kernel for the split of work between waves).
#include <type_traits>

#include "attn_device.hpp"
#include "attn_internal.h"

namespace attn {

constexpr int BWD_BN = 128;  // keys per workgroup
constexpr int BWD_BM = 64;   // queries per iteration

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
  float* dvec_out;     // D written by the D pass or the dQ kernel (same buffer as dvec)
  float* lse2_out;     // LSE * log2(e) written by the dQ kernel (same buffer as lse2)
  const float* lse;    // the forward's LSE (natural log), read by the dQ kernel
  const __bf16* out;      // the forward's output, and its rounding residual (or null)
  const __bf16* out_res;
  __bf16* dq;
  __bf16* dk;
  __bf16* dv;
  int nslots, nlogical;        // key-tile slots (dK / dV kernel)
  int nslots_q, nlogical_q;    // query-tile slots (dQ kernel)
  // dropout replay (kernels instantiated with DROP only): the forward's realisation
  uint32_t seed_lo, seed_hi, drop_thr;
  float drop_scale;
};

// Query positions [lo, hi) that see key position pk (the transpose of key_interval): from
// pk - off on with a causal mode, and only up to pk - off + window - 1 with a window; none
// for keys at or beyond len_k.
__device__ __forceinline__ void query_interval(int pk, const SeqGeom& g, int mode, int window,
                                               int& lo, int& hi) {
  lo = mode == MASK_NONE ? 0 : pk - g.off;
  hi = (mode != MASK_NONE && window > 0) ? pk - g.off + window : 0x3fffffff;
  if (pk >= g.len_k) hi = lo;
}

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
// empty rows mapped to +inf (so every recomputed P of such a row is exactly 0). One wave
// per (query token, query head).
// ---------------------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(const T* __restrict__ out,
                                                      const T* __restrict__ dout,
                                                      const float* __restrict__ lse, int total_q,
                                                      int hq, float* __restrict__ dvec,
                                                      float* __restrict__ lse2) {
  // D / 8 lanes per (token, head) row, 16 bytes of O and dO each.
  constexpr int LPR = D / 8;
  const int tid = threadIdx.x;
  const long item = (long)blockIdx.x * (256 / LPR) + tid / LPR;
  if (item >= (long)total_q * hq) return;
  const int sub = tid % LPR;
  const size_t base = (size_t)item * D + sub * 8;
  float acc = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) acc += (float)out[base + i] * (float)dout[base + i];
#pragma unroll
  for (int off = LPR / 2; off >= 1; off >>= 1) acc += __shfl_xor(acc, off, LPR);
  if (sub == 0) {
    const int t = (int)(item / hq), h = (int)(item - (long)t * hq);
    const size_t li = (size_t)h * total_q + t;
    dvec[li] = acc;
    const float l = lse[li];
    lse2[li] = (l == neg_inf()) ? __builtin_inff() : l * LOG2E;
  }
}

// ---------------------------------------------------------------------------------------
// dK / dV kernel (bf16). One workgroup = 8 waves = 128 keys of one (sequence, K/V head).
// Wave w owns key block kb = w % 4 (32 keys) and query half qh = w / 4 of every 64-query
// tile, so two waves run on each SIMD. K and V tiles stay in LDS for the whole kernel
// (DMA, swizzled rows); Q and dO tiles are DMA'd into two buffers, the next tile's load in
// flight while the current one is processed.
//   S = Q K^T, dP = dO V^T : keys on the lanes (accumulator column = key);
//   dV^T += dO^T P, dK^T += Q^T dS : P and dS are the right-hand operands as they stand,
//       dO^T / Q^T come from the tiles by transpose reads (the forward's PV access).
// The two query halves' dK / dV partials of a key block are summed through LDS at the end.
// dQ is computed by bwd_dq_kernel (query-major, no atomics).
// ---------------------------------------------------------------------------------------
template <int D>
struct BwdLds {
  static constexpr int ROWB = 2 * D;
  static constexpr int KT = BWD_BN * ROWB;            // K or V tile
  static constexpr int QT = BWD_BM * ROWB;            // Q or dO tile
  static constexpr int K_OFF = 0, V_OFF = KT, Q_OFF = 2 * KT, DO_OFF = 2 * KT + 2 * QT;
  static constexpr int VEC_OFF = 2 * KT + 4 * QT;
  static constexpr int TOTAL = VEC_OFF + 4 * BWD_BM * 4;
  // dK / dV partials of the 4 upper-half waves: 2 * (D / 32) * 16 floats per lane.
  static constexpr int RED = 4 * 2 * (D / 32) * 16 * 64 * 4;
  static_assert(RED <= VEC_OFF, "reduction area must fit in the tile area");
  static_assert(TOTAL <= LDS_BYTES, "backward tiles must fit in LDS");
};

// With DROP, Z = P * keep / (1 - p) replaces P in dV, and dP = keep / (1 - p) * (dO V^T)
// in dS = P * (dP - D); D = rowsum(dO * O) of the dropped output needs no change.
template <int D, bool DROP = false>
__global__ __launch_bounds__(512, 1) void bwd_main_kernel(BwdParams p) {
  typedef Mma<__bf16, D> M;
  typedef BwdLds<D> L;
  constexpr int ROWB = L::ROWB;
  constexpr int NDB = D / 32;
  constexpr int QREGS = D / 16;
  __shared__ __attribute__((aligned(1024))) char lds[L::TOTAL];
  char* const kt = lds + L::K_OFF;
  char* const vt = lds + L::V_OFF;
  float* const vecs = reinterpret_cast<float*>(lds + L::VEC_OFF);  // [2][lse2 | dvec][64]

  const int tid = threadIdx.x, lane = tid & 63, wave = uniform(tid >> 6);
  const int hg = lane >> 5;
  const int kb = wave & 3, qh = wave >> 2;
  const int w = xcd_logical_block(blockIdx.x, p.nlogical);
  if (w < 0) return;
  const int kvh = w / p.nslots, slot = w - kvh * p.nslots;
  const int s = seq_of_slot<BWD_BN>(p.cu_k, p.num_seqs, slot);
  const SeqGeom g = load_geom(p.cu_q, p.cu_k, s, p.mode);
  const int ntiles = (g.len_k + BWD_BN - 1) / BWD_BN;
  const int ktile = slot - (g.k_start / BWD_BN + s);
  if (ktile >= ntiles) return;
  const int k0 = ktile * BWD_BN, k1 = min(k0 + BWD_BN, g.len_k);
  const int kw0 = k0 + 32 * kb;                   // this wave's first key position
  const int kj = kw0 + (lane & 31);               // this lane's key position
  int kq_lo, kq_hi;                               // query positions that see key kj
  query_interval(kj, g, p.mode, p.window, kq_lo, kq_hi);
  const unsigned kq_width = kq_hi > kq_lo ? (unsigned)(kq_hi - kq_lo) : 0u;

  const uint32_t krs = (uint32_t)(p.hkv * D * 2);  // K/V row stride (bytes)
  const uint32_t qrs = (uint32_t)(p.hq * D * 2);   // Q/dO row stride (bytes)
  const char* kbase = reinterpret_cast<const char*>(p.k + ((size_t)g.k_start * p.hkv + kvh) * D);
  const char* vbase = reinterpret_cast<const char*>(p.v + ((size_t)g.k_start * p.hkv + kvh) * D);

  const typename M::Offsets of = M::offsets(lane);

  DmaStager<ROWB, BWD_BN, 8> kdma;
  kdma.init(wave, lane, krs);
  DmaStager<ROWB, BWD_BM, 8> qdma;
  qdma.init(wave, lane, qrs);
  kdma.issue(kbase + (size_t)k0 * krs, k1 - k0, krs, kt);
  kdma.issue(vbase + (size_t)k0 * krs, k1 - k0, krs, vt);

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
  auto tile_of = [&](int it, int& h, int& q0) {
    h = kvh * p.group + it / nqt;
    q0 = qstart + (it % nqt) * BWD_BM;
  };
  // Issue the DMA of tile `it` into buffer b and return (in registers, for tid < 64) its
  // row's LSE (base 2) and D.
  auto issue_tile = [&](int it, int b, float& l2, float& dv) {
    int h, q0;
    tile_of(it, h, q0);
    const size_t off = ((size_t)(g.q_start + q0) * p.hq + h) * D * 2;
    qdma.issue(reinterpret_cast<const char*>(p.q) + off, g.len_q - q0, qrs, lds + L::Q_OFF + b * L::QT);
    qdma.issue(reinterpret_cast<const char*>(p.dout) + off, g.len_q - q0, qrs,
               lds + L::DO_OFF + b * L::QT);
    l2 = __builtin_inff();
    dv = 0.0f;
    if (tid < BWD_BM && q0 + tid < g.len_q) {
      const size_t li = (size_t)h * p.total_q + g.q_start + q0 + tid;
      l2 = p.lse2[li];
      dv = p.dvec[li];
    }
  };
  float nl2 = 0.0f, ndv = 0.0f;
  if (niter > 0) issue_tile(0, 0, nl2, ndv);
  if (tid < BWD_BM) {
    vecs[tid] = nl2;
    vecs[BWD_BM + tid] = ndv;
  }
  wait_vmem();
  __syncthreads();

  for (int it = 0; it < niter; ++it) {
    const int b = it & 1;
    int h, q0;
    tile_of(it, h, q0);
    const int qend = min(q0 + BWD_BM, g.len_q);
    (void)h;
    if (it + 1 < niter) {
      if (tid < BWD_BM) {  // (race-exposure builds only) the slots this thread refills below
        poison4(vecs + (b ^ 1) * 2 * BWD_BM + tid);
        poison4(vecs + (b ^ 1) * 2 * BWD_BM + BWD_BM + tid);
        poison_done();
      }
      issue_tile(it + 1, b ^ 1, nl2, ndv);
    }
    const char* qtb = lds + L::Q_OFF + b * L::QT;
    const char* dotb = lds + L::DO_OFF + b * L::QT;
    const float* lse2s = vecs + b * 2 * BWD_BM;
    const float* dvs = lse2s + BWD_BM;

    const int qa = q0 + 32 * qh, qz = min(qa + 32, qend);
    const int cls = block_class(qa, qz, kw0, kw0 + 32, g, p.mode, p.window);
    if (cls != 0) {
      // Register r holds query position qa + key_of_reg(r, l / 32): allowed iff it lies in
      // this lane's key's query interval, one unsigned compare (every pair when cls == 2).
      const KeyLaneTest allowed(qa, cls, hg, kq_lo, kq_width);
      typename M::PPack pp[1], pd[1];
      // S and dP with keys on the lanes: A = Q / dO rows, B = K / V rows (all from LDS).
      f32x16 sacc = f32x16{}, dpacc = f32x16{};
      const char* qrow = qtb + 32 * qh * ROWB;
      const char* dorow = dotb + 32 * qh * ROWB;
      const char* krow = kt + 32 * kb * ROWB;
      const char* vrow = vt + 32 * kb * ROWB;
#pragma unroll
      for (int st = 0; st < QREGS; ++st) {
        const bf16x8 qa8 = *reinterpret_cast<const bf16x8*>(qrow + of.k[st]);
        const bf16x8 ka8 = *reinterpret_cast<const bf16x8*>(krow + of.k[st]);
        const bf16x8 da8 = *reinterpret_cast<const bf16x8*>(dorow + of.k[st]);
        const bf16x8 va8 = *reinterpret_cast<const bf16x8*>(vrow + of.k[st]);
        sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa8, ka8, sacc, 0, 0, 0);
        dpacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(da8, va8, dpacc, 0, 0, 0);
      }
      // P and dS; register r holds query row 32 qh + key_of_reg(r, g) of the tile. Registers
      // 4a..4a+3 hold 4 consecutive rows, so LSE2 and D arrive in 16-byte reads. The weight
      // is computed for every element and then selected: a conditional exponential became
      // one divergent branch per element, each serialising its LDS reads.
      f32x4 l4[4], d4[4];
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        l4[a] = *reinterpret_cast<const f32x4*>(lse2s + 32 * qh + 8 * a + 4 * hg);
        d4[a] = *reinterpret_cast<const f32x4*>(dvs + 32 * qh + 8 * a + 4 * hg);
      }
      // Weights and dS for MASKED blocks (some pair excluded: the lane test selects) or
      // full ones (cls == 2: every pair allowed, the test is skipped; a uniform branch
      // outside the contractions).
      auto weights = [&](auto masked) {
        constexpr bool MASKED = decltype(masked)::value;
        if constexpr (DROP) {
          const DropoutSite drop{p.seed_lo, p.seed_hi, p.drop_thr, p.drop_scale, s, h};
          // registers 4a..4a+3 hold queries qa + 8 a + 4 hg + 0..3 against key kj
          uint32_t keeps[4];
          dropout_keep_cols4(drop, (qa + 4 * hg) >> 2, kj, keeps);
#pragma unroll
          for (int a = 0; a < 4; ++a) {
            const uint32_t keep = keeps[a];
#pragma unroll
            for (int b = 0; b < 4; ++b) {
              const int r = 4 * a + b;
              const float e = fast_exp2(fmaf(sacc[r], p.c, -l4[a][b]));
              const float pv = (!MASKED || allowed.ok(r)) ? e : 0.0f;
              const bool kept = (keep >> b) & 1u;
              sacc[r] = kept ? pv * drop.scale : 0.0f;
              dpacc[r] = pv * ((kept ? dpacc[r] * drop.scale : 0.0f) - d4[a][b]);
            }
          }
        } else {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float e = fast_exp2(fmaf(sacc[r], p.c, -l4[r >> 2][r & 3]));
            const float pv = (!MASKED || allowed.ok(r)) ? e : 0.0f;
            sacc[r] = pv;
            dpacc[r] = pv * (dpacc[r] - d4[r >> 2][r & 3]);
          }
        }
      };
      if (cls == 2)
        weights(std::false_type{});
      else
        weights(std::true_type{});
      M::pack_p(sacc, pp[0]);
      M::pack_p(dpacc, pd[0]);
      // dV^T += dO^T P and dK^T += Q^T dS over this wave's 32 queries.
      M::pv(dva, pp[0], dorow, of, lane);
      M::pv(dka, pd[0], qrow, of, lane);
    }
    wait_vmem();
    if (it + 1 < niter && tid < BWD_BM) {
      vecs[(b ^ 1) * 2 * BWD_BM + tid] = nl2;
      vecs[(b ^ 1) * 2 * BWD_BM + BWD_BM + tid] = ndv;
    }
    __syncthreads();
  }

  // Sum the two query halves' partials of each key block, then store
  // dK = scale * sum dS^T Q and dV = sum P^T dO (accumulator column = key, rows = head dim).
  float* red = reinterpret_cast<float*>(lds) + (size_t)kb * (2 * NDB * 16) * 64;
  if (qh == 1) {
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        red[((0 * NDB + db) * 16 + r) * 64 + lane] = dka[db][r];
        red[((1 * NDB + db) * 16 + r) * 64 + lane] = dva[db][r];
      }
  }
  __syncthreads();
  if (qh == 0 && kj < k1) {
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        dka[db][r] += red[((0 * NDB + db) * 16 + r) * 64 + lane];
        dva[db][r] += red[((1 * NDB + db) * 16 + r) * 64 + lane];
      }
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
// dQ kernel (bf16): query-major, like the forward prefill. One workgroup = 4 waves = 128
// queries of one (sequence, query head); wave w owns 32 queries. Q and dO of the wave's
// rows are MFMA operands in registers; 64-key K and V stages are DMA'd into two buffers.
// Per stage, for each 32-key block:
//   S^T = K Q^T, dP^T = V dO^T     (queries on the lanes, as in the forward),
//   P = exp2(c S - LSE2), dS = P (dP - D)   (exactly 0 for excluded pairs and empty rows),
//   dQ^T += K^T dS^T               (the forward's PV contraction with K in place of V).
// dQ = scale * acc is written once, in the output type: no atomics, no fp32 workspace.
// ---------------------------------------------------------------------------------------
// DONLY (dropout backward only): instead of dQ, compute D = sum_j P dP of every query row
// in fp32 (dP carrying the keep / (1 - p) factor) and write it over the D that bwd_pre
// formed from the stored output. Both equal rowsum(dO * O) for the exact O; with dropout
// even a one-key row stores a rounded 1.25 v, whose rounding no longer cancels in
// dS = P (dP - D) and would move dK of such keys far beyond the gradient tolerance.
// PRE > 0 (bf16; runs before the dK/dV kernel): each query row's D = rowsum(dO * O) (with
// PRE == 2, O = the stored output plus its rounding residual) and LSE * log2(e) are formed
// here from the forward's outputs and written for the dK/dV kernel, so the backward needs
// no preprocess pass of its own.
template <int D, bool DROP = false, bool DONLY = false, int PRE = 0>
__global__ __launch_bounds__(256, 2) void bwd_dq_kernel(BwdParams p) {
  typedef Mma<__bf16, D> M;
  constexpr int BM = FWD_BM, BN = FWD_BN, ROWB = M::ROWB, TILE = BN * ROWB;
  constexpr int NDB = D / 32;
  __shared__ __attribute__((aligned(1024))) char kb0[TILE];
  __shared__ __attribute__((aligned(1024))) char kb1[TILE];
  __shared__ __attribute__((aligned(1024))) char vb0[TILE];
  __shared__ __attribute__((aligned(1024))) char vb1[TILE];

  const int tid = threadIdx.x, lane = tid & 63, wave = uniform(tid >> 6);
  const int hg = lane >> 5;
  const int w = xcd_logical_block(blockIdx.x, p.nlogical_q);
  if (w < 0) return;
  const int h = w / p.nslots_q, slot = w - h * p.nslots_q;
  const int s = seq_of_slot<BM>(p.cu_q, p.num_seqs, slot);
  const SeqGeom g = load_geom(p.cu_q, p.cu_k, s, p.mode);
  const int ntiles = (g.len_q + BM - 1) / BM;
  const int j = slot - (g.q_start / BM + s);
  if (j >= ntiles) return;
  const int tile = ntiles - 1 - j;  // latest (heaviest under causal masks) tiles first
  const int p0 = tile * BM, p1 = min(p0 + BM, g.len_q);
  const int kvh = h / p.group;
  const int wp0 = p0 + 32 * wave, wp1 = min(wp0 + 32, p1);
  const int pq = wp0 + (lane & 31);
  const bool qvalid = pq < wp1;

  bf16x8 qr[M::QREGS], dor[M::QREGS];
  const size_t qoff = ((size_t)(g.q_start + pq) * p.hq + h) * D;
  M::load_q(qr, p.q + qoff, qvalid, false, lane);
  M::load_q(dor, p.dout + qoff, qvalid, false, lane);
  const size_t li = (size_t)h * p.total_q + g.q_start + pq;
  float l2, dvl;
  if constexpr (PRE > 0) {
    bf16x8 orr[M::QREGS];
    M::load_q(orr, p.out + qoff, qvalid, false, lane);
    float part = 0.0f;
    if constexpr (PRE == 2) {
      bf16x8 rr[M::QREGS];
      M::load_q(rr, p.out_res + qoff, qvalid, false, lane);
#pragma unroll
      for (int st = 0; st < M::QREGS; ++st)
#pragma unroll
        for (int e = 0; e < 8; ++e)
          part += ((float)orr[st][e] + (float)rr[st][e]) * (float)dor[st][e];
    } else {
#pragma unroll
      for (int st = 0; st < M::QREGS; ++st)
#pragma unroll
        for (int e = 0; e < 8; ++e) part += (float)orr[st][e] * (float)dor[st][e];
    }
    const float dtot = sum_halves(part);  // lanes l and l ^ 32 hold the two row halves
    const float lv = qvalid ? p.lse[li] : neg_inf();
    l2 = lv == neg_inf() ? __builtin_inff() : lv * LOG2E;
    dvl = qvalid ? dtot : 0.0f;
    if (qvalid && lane < 32) {
      p.dvec_out[li] = dtot;
      p.lse2_out[li] = l2;
    }
  } else {
    l2 = qvalid ? p.lse2[li] : __builtin_inff();
    dvl = (!DONLY && qvalid) ? p.dvec[li] : 0.0f;
  }
  float dsum = 0.0f;  // DONLY: this lane's part of sum_j P dP
  const typename M::Offsets of = M::offsets(lane);

  int kstart, nst;
  stage_range(p0, p1, g, p.mode, p.window, BN, kstart, nst);

  const uint32_t rstride = (uint32_t)(p.hkv * D * 2);
  const char* kg = reinterpret_cast<const char*>(p.k + ((size_t)g.k_start * p.hkv + kvh) * D);
  const char* vg = reinterpret_cast<const char*>(p.v + ((size_t)g.k_start * p.hkv + kvh) * D);
  DmaStager<ROWB, BN, 4> dma;
  dma.init(wave, lane, rstride);

  f32x16 acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc[db] = f32x16{};

  int kv_lo, kv_hi;  // key positions this lane's query sees
  key_interval(pq, g, p.mode, p.window, kv_lo, kv_hi);
  const unsigned kv_width = kv_hi > kv_lo ? (unsigned)(kv_hi - kv_lo) : 0u;
  auto stage = [&](const char* kt, const char* vt, int k0) {
    const int cls = block_class(wp0, wp1, k0, k0 + BN, g, p.mode, p.window);
    if (cls == 0) return;
    const QueryLaneTest allowed(k0, cls, hg, kv_lo, kv_width);
    // Weights and dS for MASKED blocks (the lane test selects) or full ones (cls == 2: the
    // test is skipped; a uniform branch outside the contractions).
    auto weights = [&](auto masked, f32x16& sacc, const f32x16& dpacc, int kb) {
      constexpr bool MASKED = decltype(masked)::value;
      if constexpr (DROP) {
        const DropoutSite drop{p.seed_lo, p.seed_hi, p.drop_thr, p.drop_scale, s, h};
        // registers 4a..4a+3 hold keys k0 + 32 kb + 8 a + 4 hg + 0..3 against query pq
        uint32_t keeps[4];
        dropout_keep_rows4(drop, pq, (k0 + 32 * kb + 4 * hg) >> 2, keeps);
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const uint32_t keep = keeps[a];
#pragma unroll
          for (int b = 0; b < 4; ++b) {
            const int r = 4 * a + b;
            const float e = fast_exp2(fmaf(sacc[r], p.c, -l2));
            const float pv = (!MASKED || allowed.ok(kb, r)) ? e : 0.0f;
            const float dpz = ((keep >> b) & 1u) ? dpacc[r] * drop.scale : 0.0f;
            if constexpr (DONLY)
              dsum = fmaf(pv, dpz, dsum);
            else
              sacc[r] = pv * (dpz - dvl);
          }
        }
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float e = fast_exp2(fmaf(sacc[r], p.c, -l2));  // computed, then selected
          const float pv = (!MASKED || allowed.ok(kb, r)) ? e : 0.0f;
          sacc[r] = pv * (dpacc[r] - dvl);
        }
      }
    };
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      f32x16 sacc = f32x16{}, dpacc = f32x16{};
      M::qk(sacc, kt + kb * 32 * ROWB, qr, of, lane);
      M::qk(dpacc, vt + kb * 32 * ROWB, dor, of, lane);
      if (cls == 2)
        weights(std::false_type{}, sacc, dpacc, kb);
      else
        weights(std::true_type{}, sacc, dpacc, kb);
      if constexpr (!DONLY) {
        typename M::PPack pk;
        M::pack_p(sacc, pk);
        M::pv(acc, pk, kt + kb * 32 * ROWB, of, lane);
      }
    }
  };

  if (nst > 0) {
    dma.issue(kg + (size_t)kstart * rstride, g.len_k - kstart, rstride, kb0);
    dma.issue(vg + (size_t)kstart * rstride, g.len_k - kstart, rstride, vb0);
  }
  wait_vmem();
  __syncthreads();
  for (int it = 0; it < nst; it += 2) {
    const int k0 = kstart + it * BN;
    if (it + 1 < nst) {
      dma.issue(kg + (size_t)(k0 + BN) * rstride, g.len_k - k0 - BN, rstride, kb1);
      dma.issue(vg + (size_t)(k0 + BN) * rstride, g.len_k - k0 - BN, rstride, vb1);
    }
    stage(kb0, vb0, k0);
    wait_vmem();
    __syncthreads();
    if (it + 1 < nst) {
      if (it + 2 < nst) {
        dma.issue(kg + (size_t)(k0 + 2 * BN) * rstride, g.len_k - k0 - 2 * BN, rstride, kb0);
        dma.issue(vg + (size_t)(k0 + 2 * BN) * rstride, g.len_k - k0 - 2 * BN, rstride, vb0);
      }
      stage(kb1, vb1, k0 + BN);
      wait_vmem();
      __syncthreads();
    }
  }

  if constexpr (DONLY) {
    // lanes l and l ^ 32 hold the same query over different keys
    const float dtot = sum_halves(dsum);
    if (qvalid && lane < 32) p.dvec_out[li] = dtot;
    return;
  }
  // dQ = scale * acc; accumulator column = query, rows = head dim.
  if (qvalid) {
    __bf16* dst = p.dq + qoff;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int d = db * 32 + 8 * a + 4 * hg;
        M::store4(dst + d, acc[db][4 * a] * p.scale, acc[db][4 * a + 1] * p.scale,
                  acc[db][4 * a + 2] * p.scale, acc[db][4 * a + 3] * p.scale);
      }
  }
}

// ---------------------------------------------------------------------------------------
// Mask probes of the backward (see launch_mask_probe_fwd for the forward's): the kernels'
// decisions replayed with the functions they call, for one key token per wave (dK/dV
// kernel) or one query token per wave (dQ kernel). A pair enters the gradient sums iff its
// block is visited and not class 0, the lane test passes, and the query row exists (rows
// past the sequence end carry LSE = +inf, so their weights are 0).
// ---------------------------------------------------------------------------------------
__global__ void mask_probe_bwd_kv_kernel(const int32_t* cu_q, const int32_t* cu_k, int num_seqs,
                                         int mode, int window, int q0, int nq, int k0, int nk,
                                         uint8_t* bits) {
  const int u = k0 + blockIdx.x, lane = threadIdx.x, hg = lane >> 5;
  const int s = seq_of_token(cu_k, num_seqs, u);
  const SeqGeom g = load_geom(cu_q, cu_k, s, mode);
  const int kj = u - g.k_start;
  const int kt0 = (kj / BWD_BN) * BWD_BN, kt1 = min(kt0 + BWD_BN, g.len_k);
  const int kw0 = kt0 + ((kj - kt0) / 32) * 32;
  int kq_lo, kq_hi;
  query_interval(kj, g, mode, window, kq_lo, kq_hi);
  const unsigned kq_width = kq_hi > kq_lo ? (unsigned)(kq_hi - kq_lo) : 0u;
  int qlo, qhi;
  visible_queries(kt0, kt1, g, mode, window, qlo, qhi);
  const int qstart = (qlo / BWD_BM) * BWD_BM;
  const int nqt = qhi > qlo ? (qhi - qstart + BWD_BM - 1) / BWD_BM : 0;
  for (int it = 0; it < nqt; ++it) {
    const int qt0 = qstart + it * BWD_BM, qend = min(qt0 + BWD_BM, g.len_q);
    for (int qh = 0; qh < 2; ++qh) {
      const int qa = qt0 + 32 * qh, qz = min(qa + 32, qend);
      const int cls = block_class(qa, qz, kw0, kw0 + 32, g, mode, window);
      if (cls == 0) continue;
      const KeyLaneTest allowed(qa, cls, hg, kq_lo, kq_width);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int qp = qa + key_of_reg(r, hg);
        const int t = g.q_start + qp;
        if (allowed.ok(r) && qp < g.len_q && t >= q0 && t < q0 + nq)
          bits[(size_t)(t - q0) * nk + blockIdx.x] = 1;
      }
    }
  }
}

__global__ void mask_probe_bwd_q_kernel(const int32_t* cu_q, const int32_t* cu_k, int num_seqs,
                                        int mode, int window, int q0, int nq, int k0, int nk,
                                        uint8_t* bits) {
  const int t = q0 + blockIdx.x, lane = threadIdx.x, hg = lane >> 5;
  const int s = seq_of_token(cu_q, num_seqs, t);
  const SeqGeom g = load_geom(cu_q, cu_k, s, mode);
  const int pq = t - g.q_start;
  const int p0 = (pq / FWD_BM) * FWD_BM, p1 = min(p0 + FWD_BM, g.len_q);
  const int wp0 = p0 + ((pq - p0) / 32) * 32, wp1 = min(wp0 + 32, p1);
  int kstart, nst;
  stage_range(p0, p1, g, mode, window, FWD_BN, kstart, nst);
  int kv_lo, kv_hi;
  key_interval(pq, g, mode, window, kv_lo, kv_hi);
  const unsigned kv_width = kv_hi > kv_lo ? (unsigned)(kv_hi - kv_lo) : 0u;
  uint8_t* row = bits + (size_t)blockIdx.x * nk;
  for (int st = 0; st < nst; ++st) {
    const int kp = kstart + st * FWD_BN;
    const int cls = block_class(wp0, wp1, kp, kp + FWD_BN, g, mode, window);
    if (cls == 0) continue;
    const QueryLaneTest allowed(kp, cls, hg, kv_lo, kv_width);
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int u = g.k_start + kp + 32 * kb + key_of_reg(r, hg);
        if (allowed.ok(kb, r) && u >= k0 && u < k0 + nk) row[u - k0] = 1;
      }
  }
}

// The fp32 kernels' decisions: 32-key chunks against 32-query blocks (dK/dV) and 32-query
// chunks against 32-key blocks (dQ), one key / query token per wave.
__global__ void mask_probe_bwd_kv_f32_kernel(const int32_t* cu_q, const int32_t* cu_k,
                                             int num_seqs, int mode, int window, int q0, int nq,
                                             int k0, int nk, uint8_t* bits) {
  const int u = k0 + blockIdx.x, lane = threadIdx.x, hg = lane >> 5;
  const int s = seq_of_token(cu_k, num_seqs, u);
  const SeqGeom g = load_geom(cu_q, cu_k, s, mode);
  const int kj = u - g.k_start;
  const int kw0 = (kj / 32) * 32, kw1 = min(kw0 + 32, g.len_k);
  int kq_lo, kq_hi;
  query_interval(kj, g, mode, window, kq_lo, kq_hi);
  const unsigned kq_width = kq_hi > kq_lo ? (unsigned)(kq_hi - kq_lo) : 0u;
  int qlo = 0, qhi = 0;
  if (kw1 > kw0) visible_queries(kw0, kw1, g, mode, window, qlo, qhi);
  for (int qa = (qlo / 32) * 32; qa < qhi; qa += 32) {
    const int rows = min(32, g.len_q - qa);
    const int cls = block_class(qa, qa + rows, kw0, kw0 + 32, g, mode, window);
    if (cls == 0) continue;
    const KeyLaneTest allowed(qa, cls, hg, kq_lo, kq_width);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int qp = qa + key_of_reg(r, hg);
      const int t = g.q_start + qp;
      if (allowed.ok(r) && qp < g.len_q && t >= q0 && t < q0 + nq)
        bits[(size_t)(t - q0) * nk + blockIdx.x] = 1;
    }
  }
}

__global__ void mask_probe_bwd_q_f32_kernel(const int32_t* cu_q, const int32_t* cu_k,
                                            int num_seqs, int mode, int window, int q0, int nq,
                                            int k0, int nk, uint8_t* bits) {
  const int t = q0 + blockIdx.x, lane = threadIdx.x, hg = lane >> 5;
  const int s = seq_of_token(cu_q, num_seqs, t);
  const SeqGeom g = load_geom(cu_q, cu_k, s, mode);
  const int pq = t - g.q_start;
  const int qw0 = (pq / 32) * 32, qw1 = min(qw0 + 32, g.len_q);
  int kv_lo, kv_hi;
  key_interval(pq, g, mode, window, kv_lo, kv_hi);
  const unsigned kv_width = kv_hi > kv_lo ? (unsigned)(kv_hi - kv_lo) : 0u;
  int klo = 0, khi = 0;
  if (qw1 > qw0) visible_keys(qw0, qw1, g, mode, window, klo, khi);
  uint8_t* row = bits + (size_t)blockIdx.x * nk;
  for (int ka = (klo / 32) * 32; ka < khi; ka += 32) {
    const int cls = block_class(qw0, qw1, ka, ka + 32, g, mode, window);
    if (cls == 0) continue;
    const QueryLaneTest allowed(ka, cls, hg, kv_lo, kv_width);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int u = g.k_start + ka + key_of_reg(r, hg);
      if (allowed.ok(0, r) && u >= k0 && u < k0 + nk) row[u - k0] = 1;
    }
  }
}

hipError_t launch_mask_probe_bwd(const ProbeArgs& a, uint8_t* bits, hipStream_t st) {
  hipError_t e = launch_probe_zero(bits, (long)a.nq * a.nk, st);
  if (e != hipSuccess || a.nq == 0 || a.nk == 0) return e;
  if (a.unit == 3)
    hipLaunchKernelGGL(mask_probe_bwd_kv_kernel, dim3(a.nk), dim3(64), 0, st, a.cu_q, a.cu_k,
                       a.num_seqs, a.mode, a.window, a.q0, a.nq, a.k0, a.nk, bits);
  else if (a.unit == 4)
    hipLaunchKernelGGL(mask_probe_bwd_q_kernel, dim3(a.nq), dim3(64), 0, st, a.cu_q, a.cu_k,
                       a.num_seqs, a.mode, a.window, a.q0, a.nq, a.k0, a.nk, bits);
  else if (a.unit == 5)
    hipLaunchKernelGGL(mask_probe_bwd_kv_f32_kernel, dim3(a.nk), dim3(64), 0, st, a.cu_q,
                       a.cu_k, a.num_seqs, a.mode, a.window, a.q0, a.nq, a.k0, a.nk, bits);
  else
    hipLaunchKernelGGL(mask_probe_bwd_q_f32_kernel, dim3(a.nq), dim3(64), 0, st, a.cu_q,
                       a.cu_k, a.num_seqs, a.mode, a.window, a.q0, a.nq, a.k0, a.nk, bits);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------
// fp32 backward (v_mfma_f32_32x32x2_f32: exact products, fp32 accumulation), one wave per
// workgroup. Same arithmetic and mask decisions as the bf16 kernels; tiles are staged in
// LDS in the fp32 row layout of the forward (Mma<float, D>::at) by plain loads.
//   bwd_kv_f32_kernel: 32 keys of one (sequence, K/V head); for every query head of the
//     group and every 32-query block that sees them: S = Q K^T and dP = dO V^T with the
//     keys on the lanes, P and dS, then dV^T += dO^T P and dK^T += Q^T dS (the forward's
//     PV contraction over the Q / dO rows).
//   bwd_dq_f32_kernel: 32 queries of one (sequence, query head); for every 32-key block it
//     sees: S^T = K Q^T and dP^T = V dO^T with the queries on the lanes, P and dS, then
//     dQ^T += K^T dS^T.
// ---------------------------------------------------------------------------------------
template <int D>
__device__ __forceinline__ void stage_rows_f32(char* tile, const float* src, size_t row_stride,
                                               int rows, int lane) {
  // rows x D floats from src (row r at src + r * row_stride), zeros past `rows`, into the
  // swizzled fp32 row layout: lane l copies 16-byte chunks l, l + 64, ...
  typedef Mma<float, D> M;
  constexpr int CPR = D / 4;  // 16-byte chunks per row
  for (int e = lane; e < 32 * CPR; e += 64) {
    const int r = e / CPR, c = e - r * CPR;
    const f32x4 x = r < rows ? *reinterpret_cast<const f32x4*>(src + (size_t)r * row_stride + 4 * c)
                             : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    *reinterpret_cast<f32x4*>(tile + M::at(r, 4 * c)) = x;
  }
}

template <int D, bool DROP>
__global__ __launch_bounds__(64) void bwd_kv_f32_kernel(BwdParams p) {
  typedef Mma<float, D> M;
  constexpr int NDB = D / 32;
  constexpr int TB = 32 * M::ROWB;  // one 32-row tile
  __shared__ __attribute__((aligned(256))) char lds[4 * TB + 2 * 32 * 4];
  char* const kt = lds;
  char* const vt = lds + TB;
  char* const qt = lds + 2 * TB;
  char* const dot = lds + 3 * TB;
  float* const l2s = reinterpret_cast<float*>(lds + 4 * TB);
  float* const dvs = l2s + 32;
  const float* q = reinterpret_cast<const float*>(p.q);
  const float* k = reinterpret_cast<const float*>(p.k);
  const float* v = reinterpret_cast<const float*>(p.v);
  const float* dout = reinterpret_cast<const float*>(p.dout);

  const int lane = threadIdx.x, g = lane >> 5, i = lane & 31;
  const int kvh = blockIdx.y;
  // Sequence s owns key-chunk slots floor(cu_k[s] / 32) + s + j, j = its 32-key chunks.
  const int slot = blockIdx.x;
  const int s = seq_of_slot<32>(p.cu_k, p.num_seqs, slot);
  const SeqGeom geo = load_geom(p.cu_q, p.cu_k, s, p.mode);
  const int j = slot - (geo.k_start / 32 + s);
  if (j >= (geo.len_k + 31) / 32) return;
  const int kw0 = 32 * j;  // keys [kw0, kw1) of sequence s
  const int kw1 = min(kw0 + 32, geo.len_k);
  const int kj = kw0 + i;
  const bool kvalid = kj < kw1;
  int kq_lo, kq_hi;
  query_interval(kj, geo, p.mode, p.window, kq_lo, kq_hi);
  const unsigned kq_width = kq_hi > kq_lo ? (unsigned)(kq_hi - kq_lo) : 0u;
  const size_t krs = (size_t)p.hkv * D, qrs = (size_t)p.hq * D;
  stage_rows_f32<D>(kt, k + ((size_t)(geo.k_start + kw0) * p.hkv + kvh) * D, krs, kw1 - kw0, lane);
  stage_rows_f32<D>(vt, v + ((size_t)(geo.k_start + kw0) * p.hkv + kvh) * D, krs, kw1 - kw0, lane);

  f32x16 dka[NDB], dva[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    dka[db] = f32x16{};
    dva[db] = f32x16{};
  }
  int qlo = 0, qhi = 0;
  if (kw1 > kw0) visible_queries(kw0, kw1, geo, p.mode, p.window, qlo, qhi);
  const int qstart = (qlo / 32) * 32;
  for (int hh = 0; hh < p.group; ++hh) {
    const int h = kvh * p.group + hh;
    for (int qa = qstart; qa < qhi; qa += 32) {
      const int rows = min(32, geo.len_q - qa);
      __syncthreads();  // the previous block's readers are done
      stage_rows_f32<D>(qt, q + ((size_t)(geo.q_start + qa) * p.hq + h) * D, qrs, rows, lane);
      stage_rows_f32<D>(dot, dout + ((size_t)(geo.q_start + qa) * p.hq + h) * D, qrs, rows, lane);
      if (lane < 32) {
        const bool ok = lane < rows;
        const size_t li = (size_t)h * p.total_q + geo.q_start + qa + lane;
        l2s[lane] = ok ? p.lse2[li] : __builtin_inff();
        dvs[lane] = ok ? p.dvec[li] : 0.0f;
      }
      __syncthreads();
      const int cls = block_class(qa, qa + rows, kw0, kw0 + 32, geo, p.mode, p.window);
      if (cls == 0) continue;
      const KeyLaneTest allowed(qa, cls, g, kq_lo, kq_width);
      f32x16 sacc = f32x16{}, dpacc = f32x16{};
#pragma unroll 8
      for (int st = 0; st < M::QREGS; ++st) {
        const float qa_ = *reinterpret_cast<const float*>(qt + M::at(i, 2 * st + g));
        const float ka_ = *reinterpret_cast<const float*>(kt + M::at(i, 2 * st + g));
        const float da_ = *reinterpret_cast<const float*>(dot + M::at(i, 2 * st + g));
        const float va_ = *reinterpret_cast<const float*>(vt + M::at(i, 2 * st + g));
        sacc = __builtin_amdgcn_mfma_f32_32x32x2f32(qa_, ka_, sacc, 0, 0, 0);
        dpacc = __builtin_amdgcn_mfma_f32_32x32x2f32(da_, va_, dpacc, 0, 0, 0);
      }
      // register r holds query qa + key_of_reg(r, g) against key kj
      uint32_t keeps[4] = {0xFu, 0xFu, 0xFu, 0xFu};
      DropoutSite drop{p.seed_lo, p.seed_hi, p.drop_thr, p.drop_scale, s, h};
      if constexpr (DROP) dropout_keep_cols4(drop, (qa + 4 * g) >> 2, kj, keeps);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int qr = key_of_reg(r, g);
        const float e = fast_exp2(fmaf(sacc[r], p.c, -l2s[qr]));
        const float pv = allowed.ok(r) ? e : 0.0f;
        if constexpr (DROP) {
          const bool kept = (keeps[r >> 2] >> (r & 3)) & 1u;
          sacc[r] = kept ? pv * drop.scale : 0.0f;
          dpacc[r] = pv * ((kept ? dpacc[r] * drop.scale : 0.0f) - dvs[qr]);
        } else {
          sacc[r] = pv;
          dpacc[r] = pv * (dpacc[r] - dvs[qr]);
        }
      }
      typename M::PPack pp, pd;
      M::pack_p(sacc, pp);
      M::pack_p(dpacc, pd);
      M::pv(dva, pp, dot, typename M::Offsets{}, lane);
      M::pv(dka, pd, qt, typename M::Offsets{}, lane);
    }
  }
  if (kvalid) {
    float* dkrow = reinterpret_cast<float*>(p.dk) + ((size_t)(geo.k_start + kj) * p.hkv + kvh) * D;
    float* dvrow = reinterpret_cast<float*>(p.dv) + ((size_t)(geo.k_start + kj) * p.hkv + kvh) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int d = db * 32 + 8 * a + 4 * g;
        M::store4(dkrow + d, dka[db][4 * a] * p.scale, dka[db][4 * a + 1] * p.scale,
                  dka[db][4 * a + 2] * p.scale, dka[db][4 * a + 3] * p.scale);
        M::store4(dvrow + d, dva[db][4 * a], dva[db][4 * a + 1], dva[db][4 * a + 2], dva[db][4 * a + 3]);
      }
  }
}

template <int D, bool DROP>
__global__ __launch_bounds__(64) void bwd_dq_f32_kernel(BwdParams p) {
  typedef Mma<float, D> M;
  constexpr int NDB = D / 32;
  constexpr int TB = 32 * M::ROWB;
  __shared__ __attribute__((aligned(256))) char lds[2 * TB];
  char* const kt = lds;
  char* const vt = lds + TB;
  const float* q = reinterpret_cast<const float*>(p.q);
  const float* k = reinterpret_cast<const float*>(p.k);
  const float* v = reinterpret_cast<const float*>(p.v);
  const float* dout = reinterpret_cast<const float*>(p.dout);

  const int lane = threadIdx.x, g = lane >> 5;
  const int h = blockIdx.y;
  // Sequence s owns query-chunk slots floor(cu_q[s] / 32) + s + j.
  const int slot = blockIdx.x;
  const int s = seq_of_slot<32>(p.cu_q, p.num_seqs, slot);
  const SeqGeom geo = load_geom(p.cu_q, p.cu_k, s, p.mode);
  const int jq = slot - (geo.q_start / 32 + s);
  if (jq >= (geo.len_q + 31) / 32) return;
  const int qw0 = 32 * jq;  // queries [qw0, qw1) of sequence s
  const int qw1 = min(qw0 + 32, geo.len_q);
  const int pq = qw0 + (lane & 31);
  const bool qvalid = pq < qw1;
  const int kvh = h / p.group;
  typename M::QOperand qr[M::QREGS], dor[M::QREGS];
  const size_t qoff = ((size_t)(geo.q_start + pq) * p.hq + h) * D;
  M::load_q(qr, q + qoff, qvalid, false, lane);
  M::load_q(dor, dout + qoff, qvalid, false, lane);
  const size_t li = (size_t)h * p.total_q + geo.q_start + pq;
  const float l2 = qvalid ? p.lse2[li] : __builtin_inff();
  const float dvl = qvalid ? p.dvec[li] : 0.0f;
  int kv_lo, kv_hi;
  key_interval(pq, geo, p.mode, p.window, kv_lo, kv_hi);
  const unsigned kv_width = kv_hi > kv_lo ? (unsigned)(kv_hi - kv_lo) : 0u;
  int klo = 0, khi = 0;
  if (qw1 > qw0) visible_keys(qw0, qw1, geo, p.mode, p.window, klo, khi);
  const size_t krs = (size_t)p.hkv * D;
  f32x16 acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc[db] = f32x16{};
  for (int ka = (klo / 32) * 32; ka < khi; ka += 32) {
    const int rows = min(32, geo.len_k - ka);
    __syncthreads();
    stage_rows_f32<D>(kt, k + ((size_t)(geo.k_start + ka) * p.hkv + kvh) * D, krs, rows, lane);
    stage_rows_f32<D>(vt, v + ((size_t)(geo.k_start + ka) * p.hkv + kvh) * D, krs, rows, lane);
    __syncthreads();
    const int cls = block_class(qw0, qw1, ka, ka + 32, geo, p.mode, p.window);
    if (cls == 0) continue;
    const QueryLaneTest allowed(ka, cls, g, kv_lo, kv_width);
    f32x16 sacc = f32x16{}, dpacc = f32x16{};
    M::qk(sacc, kt, qr, typename M::Offsets{}, lane);
    M::qk(dpacc, vt, dor, typename M::Offsets{}, lane);
    uint32_t keeps[4] = {0xFu, 0xFu, 0xFu, 0xFu};
    DropoutSite drop{p.seed_lo, p.seed_hi, p.drop_thr, p.drop_scale, s, h};
    if constexpr (DROP) dropout_keep_rows4(drop, pq, (ka + 4 * g) >> 2, keeps);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float e = fast_exp2(fmaf(sacc[r], p.c, -l2));
      const float pv = allowed.ok(0, r) ? e : 0.0f;
      const float dpz =
          DROP ? (((keeps[r >> 2] >> (r & 3)) & 1u) ? dpacc[r] * drop.scale : 0.0f) : dpacc[r];
      sacc[r] = pv * (dpz - dvl);
    }
    typename M::PPack pk;
    M::pack_p(sacc, pk);
    M::pv(acc, pk, kt, typename M::Offsets{}, lane);
  }
  if (qvalid) {
    float* dst = reinterpret_cast<float*>(p.dq) + qoff;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int d = db * 32 + 8 * a + 4 * g;
        M::store4(dst + d, acc[db][4 * a] * p.scale, acc[db][4 * a + 1] * p.scale,
                  acc[db][4 * a + 2] * p.scale, acc[db][4 * a + 3] * p.scale);
      }
  }
}

// ---------------------------------------------------------------------------------------
// Launch
// ---------------------------------------------------------------------------------------
size_t bwd_workspace_bytes(int total_q, int hq, int d) {
  (void)d;
  const size_t vec = (size_t)total_q * hq * sizeof(float);
  return 2 * (((vec + 255) / 256) * 256);
}

template <typename T, int D>
static hipError_t bwd_typed(const BwdArgs& a, void* ws, hipStream_t st) {
  const FwdArgs& f = a.f;
  const size_t vecb = (((size_t)f.total_q * f.hq * sizeof(float) + 255) / 256) * 256;
  float* dvec = static_cast<float*>(ws);
  float* lse2 = reinterpret_cast<float*>(static_cast<char*>(ws) + vecb);
  const long items = (long)f.total_q * f.hq;
  const bool drop = f.drop_thr > 0;
  // bf16 without dropout, or with the forward's output residual: the dQ kernel runs first
  // and forms D and LSE * log2(e) itself (no preprocess pass); the dK/dV kernel follows.
  const bool fused = std::is_same<T, __bf16>::value && (!drop || a.out_res != nullptr);
  if (items > 0 && !fused) {
    hipLaunchKernelGGL((bwd_pre_kernel<T, D>),
                       dim3((unsigned)((items + 256 / (D / 8) - 1) / (256 / (D / 8)))),
                       dim3(256), 0, st, static_cast<const T*>(a.out),
                       static_cast<const T*>(a.dout), a.lse, f.total_q, f.hq, dvec, lse2);
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
  p.dq = static_cast<__bf16*>(a.dq);
  p.dk = static_cast<__bf16*>(a.dk);
  p.dv = static_cast<__bf16*>(a.dv);
  p.nslots = f.total_k / BWD_BN + f.num_seqs;
  p.nlogical = p.nslots * f.hkv;
  p.nslots_q = f.total_q / FWD_BM + f.num_seqs;
  p.nlogical_q = p.nslots_q * f.hq;
  p.seed_lo = (uint32_t)f.seed;
  p.seed_hi = (uint32_t)(f.seed >> 32);
  p.drop_thr = f.drop_thr;
  p.drop_scale = f.drop_scale;
  p.dvec_out = dvec;
  p.lse2_out = lse2;
  p.lse = a.lse;
  p.out = static_cast<const __bf16*>(a.out);
  p.out_res = static_cast<const __bf16*>(a.out_res);
  if constexpr (std::is_same<T, float>::value) {
    // fp32: one wave per 32-key / 32-query chunk slot (D = rowsum(dO * O) from the fp32
    // output is exact enough here: no separate D pass).
    const int kslots = f.total_k / 32 + f.num_seqs, qslots = f.total_q / 32 + f.num_seqs;
    if (f.total_k > 0) {
      if (drop)
        hipLaunchKernelGGL((bwd_kv_f32_kernel<D, true>), dim3(kslots, f.hkv), dim3(64), 0, st, p);
      else
        hipLaunchKernelGGL((bwd_kv_f32_kernel<D, false>), dim3(kslots, f.hkv), dim3(64), 0, st, p);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    if (f.total_q > 0) {
      if (drop)
        hipLaunchKernelGGL((bwd_dq_f32_kernel<D, true>), dim3(qslots, f.hq), dim3(64), 0, st, p);
      else
        hipLaunchKernelGGL((bwd_dq_f32_kernel<D, false>), dim3(qslots, f.hq), dim3(64), 0, st, p);
    }
    return hipGetLastError();
  }
  if (fused) {
    if (f.total_q > 0) {
      const int grid = ((p.nlogical_q + 7) / 8) * 8;
      if (drop)
        hipLaunchKernelGGL((bwd_dq_kernel<D, true, false, 2>), dim3(grid), dim3(256), 0, st, p);
      else if (a.out_res != nullptr)
        hipLaunchKernelGGL((bwd_dq_kernel<D, false, false, 2>), dim3(grid), dim3(256), 0, st, p);
      else
        hipLaunchKernelGGL((bwd_dq_kernel<D, false, false, 1>), dim3(grid), dim3(256), 0, st, p);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    if (f.total_k > 0) {
      const int grid = ((p.nlogical + 7) / 8) * 8;
      if (drop)
        hipLaunchKernelGGL((bwd_main_kernel<D, true>), dim3(grid), dim3(512), 0, st, p);
      else
        hipLaunchKernelGGL((bwd_main_kernel<D>), dim3(grid), dim3(512), 0, st, p);
    }
    return hipGetLastError();
  }
  // Dropout without the residual: D = sum_j P dP needs the unrounded output, so a pass of
  // its own computes it exactly before the dK/dV and dQ kernels.
  if (drop && f.total_q > 0) {
    const int grid = ((p.nlogical_q + 7) / 8) * 8;
    hipLaunchKernelGGL((bwd_dq_kernel<D, true, true>), dim3(grid), dim3(256), 0, st, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (f.total_k > 0) {
    const int grid = ((p.nlogical + 7) / 8) * 8;
    if (drop)
      hipLaunchKernelGGL((bwd_main_kernel<D, true>), dim3(grid), dim3(512), 0, st, p);
    else
      hipLaunchKernelGGL((bwd_main_kernel<D>), dim3(grid), dim3(512), 0, st, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (f.total_q > 0) {
    const int grid = ((p.nlogical_q + 7) / 8) * 8;
    if (drop)
      hipLaunchKernelGGL((bwd_dq_kernel<D, true>), dim3(grid), dim3(256), 0, st, p);
    else
      hipLaunchKernelGGL((bwd_dq_kernel<D>), dim3(grid), dim3(256), 0, st, p);
  }
  return hipGetLastError();
}

hipError_t launch_bwd(const BwdArgs& a, void* ws, hipStream_t st) {
  if (a.f.dtype == 0)
    return a.f.d == 64 ? bwd_typed<__bf16, 64>(a, ws, st) : bwd_typed<__bf16, 128>(a, ws, st);
  return a.f.d == 64 ? bwd_typed<float, 64>(a, ws, st) : bwd_typed<float, 128>(a, ws, st);
}

}  // namespace attn
