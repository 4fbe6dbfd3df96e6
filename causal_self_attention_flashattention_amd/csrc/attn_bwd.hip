// Attention backward with recomputation (gfx950): three kernels on one stream.
//
// The math is eqs. (13)-(19) of the CS336 Assignment 2 (systems) handout, §4.1 ("backward
// pass with recomputation"): S = scale Q K^T, P_ij = exp(S_ij - L_i), dV = P^T dO,
// dP = dO V^T, dS_ij = P_ij (dP_ij - D_i), dQ = scale dS K, dK = scale dS^T Q, with
// D = rowsum(O o dO) computed first.  Following the key idea of the handout's tiled backward
// (§4.2.3), P is recomputed twice -- once in a kernel that owns key tiles and accumulates dK
// and dV, once in a kernel that owns query tiles and accumulates dQ -- so no workgroup ever
// writes another's output and no atomics are needed (results are bitwise reproducible).
//
//  rowdot_kernel  D_i = sum_c O_ic dO_ic (fp32), one pass over O and dO, bandwidth bound.
//  dkdv_kernel    per (head, 32*NW keys): S and dP with queries on MFMA rows and keys on
//                 columns, so P and dS come out of the accumulators already shaped as the B
//                 operand of dV^T += dO^T P and dK^T += Q^T dS (dO^T, Q^T by LDS transpose reads).
//  dq_kernel      per (head, 32*NW queries): S^T and dP^T with keys on rows, so dS^T feeds
//                 dQ^T += K^T dS^T directly.
// The causal / key-padding mask is regenerated from indices; whole blocks above the diagonal or
// past the key length are skipped.
#include "attn_device.h"
#include "launch.h"

namespace attn {

// ------------------------------------------------------------------------------------------
// D = rowsum(O o dO)

template <typename T, int D>
__global__ __launch_bounds__(256) void rowdot_kernel(const T* __restrict__ O, const T* __restrict__ dO,
                                                     float* __restrict__ Dv, int rows) {
  constexpr int EPC = 16 / (int)sizeof(T);  // elements per 16-byte chunk
  constexpr int CPR = D / EPC;              // chunks per row
  constexpr int TPR = CPR <= 1 ? 1 : CPR <= 2 ? 2 : CPR <= 4 ? 4 : CPR <= 8 ? 8 : CPR <= 16 ? 16 : 32;
  static_assert(D % EPC == 0 && CPR <= 32, "unsupported head dim");
  constexpr int RPB = 256 / TPR;  // rows per block per step
  const int sub = threadIdx.x % TPR;
  for (int row = blockIdx.x * RPB + threadIdx.x / TPR; row < rows; row += gridDim.x * RPB) {
    float acc = 0.f;
    if (sub < CPR) {
      const uint4 a = *reinterpret_cast<const uint4*>(O + (size_t)row * D + sub * EPC);
      const uint4 g = *reinterpret_cast<const uint4*>(dO + (size_t)row * D + sub * EPC);
      T av[EPC], gv[EPC];
      __builtin_memcpy(av, &a, 16);
      __builtin_memcpy(gv, &g, 16);
#pragma unroll
      for (int i = 0; i < EPC; ++i) acc += (float)av[i] * (float)gv[i];
    }
#pragma unroll
    for (int m = TPR / 2; m > 0; m >>= 1) acc += __shfl_xor(acc, m, TPR);
    if (sub == 0) Dv[row] = acc;
  }
}

// ------------------------------------------------------------------------------------------
// dK, dV: one workgroup per (head, 32*NW keys); loop over query tiles of BQ rows.

template <typename T, int D, int NW, int BQ>
__global__ __launch_bounds__(NW * 64) void dkdv_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V, const T* __restrict__ dO,
    const float* __restrict__ Lse, const float* __restrict__ Dv, T* __restrict__ dK, T* __restrict__ dV,
    int BH, int H, int N, int causal, float scale, float scale_log2, const int32_t* __restrict__ kv_len) {
  using M = Mfma<T>;
  constexpr int NT = NW * 64;
  constexpr int KT = 32 * NW;  // keys per workgroup
  constexpr int DP = (D + 31) / 32 * 32;
  constexpr int NDB = DP / 32;
  constexpr int KS = D / M::KSTEP;
  constexpr int NQB = BQ / 32;
  constexpr int LD = DP + 16 / (int)sizeof(T);

  __shared__ __attribute__((aligned(16))) char smem[2 * BQ * LD * sizeof(T) + 2 * BQ * sizeof(float)];
  lds_t* qtile = (lds_t*)smem;
  lds_t* otile = qtile + BQ * LD * sizeof(T);  // dO tile
  float* lrow = reinterpret_cast<float*>(smem + 2 * BQ * LD * sizeof(T));  // L * log2(e), per query
  float* drow = lrow + BQ;                                                 // D, per query

  const int TK = (N + KT - 1) / KT;
  const int logical = xcd_logical_block(BH * TK);
  if (logical < 0) return;
  const int bh = logical / TK;
  const int kt = logical % TK;  // low key tiles see the most queries under causal masking
  const int b = bh / H;
  int kv = N;
  if (kv_len) kv = min(max(kv_len[b], 1), N);

  const size_t base = (size_t)bh * N * D;
  Q += base; K += base; V += base; dO += base; dK += base; dV += base;
  Lse += (size_t)bh * N;
  Dv += (size_t)bh * N;

  const int w = threadIdx.x >> 6, l = lane_id(), half = l >> 5, col = l & 31;
  const int k0 = kt * KT;
  const int kw = k0 + 32 * w;  // first key of this wave
  const int key = kw + col;    // this lane's key
  const bool wave_live = kw < kv;

  f32x16 dk[NDB], dv[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) { dk[i] = f32x16{}; dv[i] = f32x16{}; }

  if (k0 < kv) {
    typename M::frag kf[KS], vf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      kf[ks] = M::load_global(K + (size_t)min(key, N - 1) * D, ks * M::KSTEP, key < N);
      vf[ks] = M::load_global(V + (size_t)min(key, N - 1) * D, ks * M::KSTEP, key < N);
    }
    const int TQ = (N + BQ - 1) / BQ;
    const int qt0 = causal ? k0 / BQ : 0;

    TileCopy<T, BQ, D, LD, NT> qc, oc;
    zero_pad_cols<T, BQ, D, LD, DP, NT>(qtile);
    zero_pad_cols<T, BQ, D, LD, DP, NT>(otile);
    qc.load(Q + (size_t)qt0 * BQ * D, N - qt0 * BQ);
    oc.load(dO + (size_t)qt0 * BQ * D, N - qt0 * BQ);
    for (int qt = qt0; qt < TQ; ++qt) {
      const int q0 = qt * BQ;
      __syncthreads();
      qc.store(qtile);
      oc.store(otile);
      for (int i = threadIdx.x; i < BQ; i += NT) {
        const int qq = q0 + i;
        lrow[i] = qq < N ? Lse[qq] * kLog2e : 0.f;
        drow[i] = qq < N ? Dv[qq] : 0.f;
      }
      __syncthreads();
      if (qt + 1 < TQ) {
        qc.load(Q + (size_t)(qt + 1) * BQ * D, N - (qt + 1) * BQ);
        oc.load(dO + (size_t)(qt + 1) * BQ * D, N - (qt + 1) * BQ);
      }
      if (!wave_live) continue;
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) {
        const int qb0 = q0 + qb * 32;
        if (qb0 >= N || (causal && qb0 + 31 < kw)) continue;  // past the end, or all queries before this wave's keys
        f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          s = M::mma(M::frag_direct(qtile, LD, qb * 32 * LD + ks * M::KSTEP), kf[ks], s);
          dp = M::mma(M::frag_direct(otile, LD, qb * 32 * LD + ks * M::KSTEP), vf[ks], dp);
        }
        const bool need_mask = (causal && kw + 31 > qb0) || (kw + 32 > kv) || (qb0 + 32 > N);
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const int r0 = qb * 32 + 8 * m + 4 * half;
          const float4 lv = *reinterpret_cast<const float4*>(lrow + r0);
          const float4 dd = *reinterpret_cast<const float4*>(drow + r0);
          const float la[4] = {lv.x, lv.y, lv.z, lv.w};
          const float da[4] = {dd.x, dd.y, dd.z, dd.w};
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int e = 4 * m + r;
            float p = fast_exp2(s[e] * scale_log2 - la[r]);
            if (need_mask) {
              const int qq = q0 + r0 + r;
              if ((causal && key > qq) || key >= kv || qq >= N) p = 0.f;
            }
            s[e] = p;
            dp[e] = p * (dp[e] - da[r]);
          }
        }
#pragma unroll
        for (int c = 0; c < M::CALLS32; ++c) {
          const typename M::frag pf = M::acc_frag(s, c);
          const typename M::frag sf = M::acc_frag(dp, c);
#pragma unroll
          for (int db = 0; db < NDB; ++db) {
            dv[db] = M::mma(M::frag_trans(otile, LD, qb * 32 * LD + db * 32, c), pf, dv[db]);
            dk[db] = M::mma(M::frag_trans(qtile, LD, qb * 32 * LD + db * 32, c), sf, dk[db]);
          }
        }
      }
    }
  }

  if (key < N) {
    T* krow = dK + (size_t)key * D;
    T* vrow = dV + (size_t)key * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int d0 = db * 32 + 8 * m + 4 * half;
        if (D % 32 == 0 || d0 < D) {
          T kk[4], vv[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            kk[r] = (T)(dk[db][4 * m + r] * scale);
            vv[r] = (T)dv[db][4 * m + r];
          }
          if constexpr (sizeof(T) == 2) {
            uint2 u;
            __builtin_memcpy(&u, kk, 8);
            *reinterpret_cast<uint2*>(krow + d0) = u;
            __builtin_memcpy(&u, vv, 8);
            *reinterpret_cast<uint2*>(vrow + d0) = u;
          } else {
            uint4 u;
            __builtin_memcpy(&u, kk, 16);
            *reinterpret_cast<uint4*>(krow + d0) = u;
            __builtin_memcpy(&u, vv, 16);
            *reinterpret_cast<uint4*>(vrow + d0) = u;
          }
        }
      }
  }
}

// ------------------------------------------------------------------------------------------
// dQ: one workgroup per (head, 32*NW queries); loop over key tiles of BK rows.

template <typename T, int D, int NW, int BK>
__global__ __launch_bounds__(NW * 64) void dq_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V, const T* __restrict__ dO,
    const float* __restrict__ Lse, const float* __restrict__ Dv, T* __restrict__ dQ, int BH, int H, int N,
    int causal, float scale, float scale_log2, const int32_t* __restrict__ kv_len) {
  using M = Mfma<T>;
  constexpr int NT = NW * 64;
  constexpr int QT = 32 * NW;
  constexpr int DP = (D + 31) / 32 * 32;
  constexpr int NDB = DP / 32;
  constexpr int KS = D / M::KSTEP;
  constexpr int NB = BK / 32;
  constexpr int LD = DP + 16 / (int)sizeof(T);

  __shared__ __attribute__((aligned(16))) char smem[2 * BK * LD * sizeof(T)];
  lds_t* ktile = (lds_t*)smem;
  lds_t* vtile = ktile + BK * LD * sizeof(T);

  const int TQ = (N + QT - 1) / QT;
  const int logical = xcd_logical_block(BH * TQ);
  if (logical < 0) return;
  const int bh = logical / TQ;
  const int qt = TQ - 1 - logical % TQ;
  const int b = bh / H;
  int kv = N;
  if (kv_len) kv = min(max(kv_len[b], 1), N);

  const size_t base = (size_t)bh * N * D;
  Q += base; K += base; V += base; dO += base; dQ += base;
  Lse += (size_t)bh * N;
  Dv += (size_t)bh * N;

  const int w = threadIdx.x >> 6, l = lane_id(), half = l >> 5, col = l & 31;
  const int q0 = qt * QT;
  const int qw = q0 + 32 * w;
  const int q = qw + col;
  const int qw_last = min(qw + 31, N - 1);

  int kend = kv;
  if (causal) kend = min(kend, q0 + QT);
  const int nkt = (kend + BK - 1) / BK;

  typename M::frag qf[KS], of[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    qf[ks] = M::load_global(Q + (size_t)min(q, N - 1) * D, ks * M::KSTEP, q < N);
    of[ks] = M::load_global(dO + (size_t)min(q, N - 1) * D, ks * M::KSTEP, q < N);
  }
  const float lq = q < N ? Lse[q] * kLog2e : 0.f;
  const float dq_ = q < N ? Dv[q] : 0.f;

  f32x16 acc[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) acc[i] = f32x16{};

  TileCopy<T, BK, D, LD, NT> kc, vc;
  zero_pad_cols<T, BK, D, LD, DP, NT>(ktile);
  kc.load(K, kend);
  vc.load(V, kend);
  for (int kt = 0; kt < nkt; ++kt) {
    __syncthreads();
    kc.store(ktile);
    vc.store(vtile);
    __syncthreads();
    if (kt + 1 < nkt) {
      kc.load(K + (size_t)(kt + 1) * BK * D, kend - (kt + 1) * BK);
      vc.load(V + (size_t)(kt + 1) * BK * D, kend - (kt + 1) * BK);
    }
    if (qw >= N) continue;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int kb0 = kt * BK + nb * 32;
      if (kb0 >= kend || (causal && kb0 > qw_last)) continue;
      f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        s = M::mma(M::frag_direct(ktile, LD, nb * 32 * LD + ks * M::KSTEP), qf[ks], s);
        dp = M::mma(M::frag_direct(vtile, LD, nb * 32 * LD + ks * M::KSTEP), of[ks], dp);
      }
      const bool need_mask = (causal && kb0 + 31 > qw) || (kb0 + 32 > kv);
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        float p = fast_exp2(s[e] * scale_log2 - lq);
        if (need_mask) {
          const int kk = kb0 + acc_row(e, half);
          if ((causal && kk > q) || kk >= kv) p = 0.f;
        }
        dp[e] = p * (dp[e] - dq_);
      }
#pragma unroll
      for (int c = 0; c < M::CALLS32; ++c) {
        const typename M::frag sf = M::acc_frag(dp, c);
#pragma unroll
        for (int db = 0; db < NDB; ++db)
          acc[db] = M::mma(M::frag_trans(ktile, LD, nb * 32 * LD + db * 32, c), sf, acc[db]);
      }
    }
  }

  if (q < N) {
    T* row = dQ + (size_t)q * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int d0 = db * 32 + 8 * m + 4 * half;
        if (D % 32 == 0 || d0 < D) {
          T v4[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) v4[r] = (T)(acc[db][4 * m + r] * scale);
          if constexpr (sizeof(T) == 2) {
            uint2 u;
            __builtin_memcpy(&u, v4, 8);
            *reinterpret_cast<uint2*>(row + d0) = u;
          } else {
            uint4 u;
            __builtin_memcpy(&u, v4, 16);
            *reinterpret_cast<uint4*>(row + d0) = u;
          }
        }
      }
  }
}

// ------------------------------------------------------------------------------------------
// launchers

template <typename T, int D>
static hipError_t launch_rowdot_t(const Problem& p, const void* O, const void* dO, float* Dv, hipStream_t s) {
  const int rows = p.B * p.H * p.N;
  constexpr int CPR = D * (int)sizeof(T) / 16;
  constexpr int TPR = CPR <= 1 ? 1 : CPR <= 2 ? 2 : CPR <= 4 ? 4 : CPR <= 8 ? 8 : CPR <= 16 ? 16 : 32;
  constexpr int RPB = 256 / TPR;
  int grid = (rows + RPB - 1) / RPB;
  if (grid > 256 * 16) grid = 256 * 16;
  hipLaunchKernelGGL((rowdot_kernel<T, D>), dim3(grid), dim3(256), 0, s, (const T*)O, (const T*)dO, Dv, rows);
  return hipGetLastError();
}

template <typename T, int D, int NW, int BQ>
static hipError_t launch_dkdv_t(const Problem& p, const void* Q, const void* K, const void* V, const void* dO,
                                const float* L, const float* Dv, void* dK, void* dV, hipStream_t s) {
  constexpr int KT = 32 * NW;
  const int TK = (p.N + KT - 1) / KT;
  const int nlog = p.B * p.H * TK;
  const int grid = (nlog + 7) / 8 * 8;
  hipLaunchKernelGGL((dkdv_kernel<T, D, NW, BQ>), dim3(grid), dim3(NW * 64), 0, s, (const T*)Q, (const T*)K,
                     (const T*)V, (const T*)dO, L, Dv, (T*)dK, (T*)dV, p.B * p.H, p.H, p.N, p.causal, p.scale,
                     p.scale * kLog2e, p.kv_len);
  return hipGetLastError();
}

template <typename T, int D, int NW, int BK>
static hipError_t launch_dq_t(const Problem& p, const void* Q, const void* K, const void* V, const void* dO,
                              const float* L, const float* Dv, void* dQ, hipStream_t s) {
  constexpr int QT = 32 * NW;
  const int TQ = (p.N + QT - 1) / QT;
  const int nlog = p.B * p.H * TQ;
  const int grid = (nlog + 7) / 8 * 8;
  hipLaunchKernelGGL((dq_kernel<T, D, NW, BK>), dim3(grid), dim3(NW * 64), 0, s, (const T*)Q, (const T*)K,
                     (const T*)V, (const T*)dO, L, Dv, (T*)dQ, p.B * p.H, p.H, p.N, p.causal, p.scale,
                     p.scale * kLog2e, p.kv_len);
  return hipGetLastError();
}

bool bwd_supported(int dtype, int d) { return fwd_supported(dtype, d); }

#define ATTN_BWD_CASES(X)                                     \
  X(__bf16, kBF16, 16) X(__bf16, kBF16, 32) X(__bf16, kBF16, 64) \
  X(__bf16, kBF16, 80) X(__bf16, kBF16, 128) X(float, kF32, 16) \
  X(float, kF32, 32) X(float, kF32, 64) X(float, kF32, 80) X(float, kF32, 128)

hipError_t launch_rowdot(int dtype, const Problem& p, const void* O, const void* dO, float* Dv, hipStream_t s) {
#define X(T, DT, DD) \
  if (dtype == DT && p.d == DD) return launch_rowdot_t<T, DD>(p, O, dO, Dv, s);
  ATTN_BWD_CASES(X)
#undef X
  return hipErrorInvalidValue;
}

hipError_t launch_dkdv(int dtype, const Problem& p, const void* Q, const void* K, const void* V, const void* dO,
                       const float* L, const float* Dv, void* dK, void* dV, hipStream_t s) {
#define X(T, DT, DD) \
  if (dtype == DT && p.d == DD) return launch_dkdv_t<T, DD, 4, (DT == kBF16 ? 64 : 32)>(p, Q, K, V, dO, L, Dv, dK, dV, s);
  ATTN_BWD_CASES(X)
#undef X
  return hipErrorInvalidValue;
}

hipError_t launch_dq(int dtype, const Problem& p, const void* Q, const void* K, const void* V, const void* dO,
                     const float* L, const float* Dv, void* dQ, hipStream_t s) {
#define X(T, DT, DD) \
  if (dtype == DT && p.d == DD) return launch_dq_t<T, DD, 4, (DT == kBF16 ? 64 : 32)>(p, Q, K, V, dO, L, Dv, dQ, s);
  ATTN_BWD_CASES(X)
#undef X
  return hipErrorInvalidValue;
}

}  // namespace attn
