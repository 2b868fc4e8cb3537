// Chunked gated-delta-rule replay on the gfx950 matrix cores.
//
// The per-token recurrence ("SuffixReplay", Eq. 4 with decay + rank-one
// erase; "Tail-Replay", section 2)
//     S_t = a_t S_{t-1} (I - b_t k_t k_t^T) + b_t v_t k_t^T,   o_t = S_t q_t
// is evaluated 64 tokens at a time.  Within a chunk (g_t = log a_t,
// G_t = sum_{s<=t} g_s, everything below is exact algebra of the recurrence):
//     A[t][j] = b_t e^{G_t-G_j} (k_t . k_j), j < t        (strictly lower)
//     Tm      = (I + A)^{-1}
//     W       = Tm diag(b e^G) K,   U~ = Tm diag(b) V
//     U       = U~ - W S^T                                  (needs the carry)
//     O       = diag(e^G) Q S^T + (P o Q K^T) U,  P[t][j] = e^{G_t-G_j}, j<=t
//     S^T    <- e^{G_C} S^T + K^T diag(e^{G_C-G}) U
// Erase-free mode (scalar decay only): A = 0, U = diag(b) V.
//
// Layout of the work: one workgroup (4 waves) per (sequence, value head)
// walks that sequence's chunks in order.  The transposed state S^T (d_k x
// d_v, fp32) stays in matrix-core accumulator registers for the whole
// sequence; wave w owns value columns [w*D/4, (w+1)*D/4).  Accumulator tiles
// of S^T, U and O feed the next products directly as B operands: two
// vertically adjacent 16x16 accumulator tiles hold, per lane, the 8 k-slots
// {4g..4g+3, 16+4g..16+4g+3} (g = lane/16) of a K = 32 operand, and the A
// operand is read from LDS in the same k order.  Operands are fp16 (bf16
// inputs convert exactly); accumulation and the state are fp32.
// The 64x64 triangular inverse is done in fp32 in LDS by blocked forward
// substitution (16x16 diagonal blocks, then block columns).
#include "sr_common.hpp"
#include "sr_internal.hpp"

namespace sr {

namespace {

constexpr int kC = 64;          // chunk length (tokens)
constexpr int kThreads = 256;   // 4 waves
constexpr int kTS = kC + 8;     // fp16 row stride of [.][64] LDS tiles
constexpr int kAS = kC + 4;     // fp32 row stride of the 64x64 fp32 tiles

template <int D>
struct ChunkSmem {
  static constexpr int kWS = D + 8;  // fp16 row stride of the [64][D] W tile
  _Float16 kt[D * kTS];              // K^T of the chunk  [j][t]
  _Float16 vt[D * kTS];              // V^T of the chunk  [i][t]
  union {
    float a[kC * kAS];               // A (fp32)          [t][j]
    _Float16 w[kC * kWS];            // -W                [t][j]
  } aw;
  union {
    float tm[kC * kAS];              // (I+A)^-1 (fp32) while solving
    struct {
      _Float16 tb[kC * kTS];         // Tm diag(b)
      _Float16 tbg[kC * kTS];        // Tm diag(b e^G)
    } t16;
    _Float16 pqk[kC * kTS];          // P o (Q K^T)
  } tt;
  float gcum[kC];                    // G_t
  float gam[kC];                     // e^{G_t}
  float dec[kC];                     // e^{G_C - G_t}
  float beta[kC];                    // b_t (0 past the end of the sequence)
  float bg[kC];                      // b_t e^{G_t}
};

// 16x16 tile MFMA over K = 32 with both operands 8 consecutive fp16 in LDS.
__device__ __forceinline__ f16x8 lds8(const _Float16* p) {
  return *reinterpret_cast<const f16x8*>(p);
}
__device__ __forceinline__ f16x4 lds4(const _Float16* p) {
  return *reinterpret_cast<const f16x4*>(p);
}
// A operand in the permuted k order {4g..4g+3, 16+4g..16+4g+3} of a 32-wide
// k block starting at p (p already offset by the row).
__device__ __forceinline__ f16x8 lds_perm(const _Float16* p, int lg) {
  return cat44(lds4(p + 4 * lg), lds4(p + 16 + 4 * lg));
}

template <int D, typename TI, typename TO, bool ERASE>
__global__ __launch_bounds__(kThreads, 2) void gdn_chunk_kernel(GdnArgs a) {
  constexpr int IW = D / 4;       // value columns per wave
  constexpr int NIT = IW / 16;    // 16-wide value tiles per wave
  constexpr int NJT = D / 16;     // 16-wide key tiles
  constexpr int NKJ = D / 32;     // K = 32 steps over the key dimension
  constexpr int kWS = ChunkSmem<D>::kWS;
  static_assert(NIT >= 1, "D too small");

  __shared__ ChunkSmem<D> sm;

  const int n = blockIdx.x / a.h_v;
  const int h = blockIdx.x % a.h_v;
  const int g = h / (a.h_v / a.h_k);
  const int tid = threadIdx.x;
  const int w = tid / kWave;
  const int l = tid % kWave;
  const int lr = l % 16;
  const int lg = l / 16;
  const bool want_o = a.o != nullptr;
  const size_t qk_stride = static_cast<size_t>(a.h_k) * D;   // per token
  const size_t v_stride = static_cast<size_t>(a.h_v) * D;
  const char* qg = static_cast<const char*>(a.q) + static_cast<size_t>(g) * D * Ld8<TI>::kBytes;
  const char* kg = static_cast<const char*>(a.k) + static_cast<size_t>(g) * D * Ld8<TI>::kBytes;
  const char* vg = static_cast<const char*>(a.v) + static_cast<size_t>(h) * D * Ld8<TI>::kBytes;
  constexpr int EB = Ld8<TI>::kBytes;

  // S^T accumulators: tile (jt, it) covers key rows 16jt.., value columns
  // w*IW + 16it..; lane holds column lr, rows 4lg..4lg+3.
  f32x4 S[NJT][NIT];
  const size_t sbase = (static_cast<size_t>(n) * a.h_v + h) * D * D;
#pragma unroll
  for (int jt = 0; jt < NJT; ++jt)
#pragma unroll
    for (int it = 0; it < NIT; ++it)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int j = 16 * jt + 4 * lg + r;
        const int i = w * IW + 16 * it + lr;
        S[jt][it][r] = a.s0 ? a.s0[sbase + static_cast<size_t>(j) * D + i] : 0.0f;
      }

  const int t_begin = a.cu[n];
  const int t_end = a.cu[n + 1];

  for (int c0 = t_begin; c0 < t_end; c0 += kC) {
    const int nv = min(kC, t_end - c0);

    // ---- stage K^T, V^T (fp16) and the gate scalars ----------------------
    for (int item = tid; item < (kC / 2) * (D / 8); item += kThreads) {
      const int p = item / (D / 8);
      const int jc = item % (D / 8);
      const int t = 2 * p;
      f16x8 r0 = {}, r1 = {};
      if (t < nv) r0 = Ld8<TI>::load(kg + ((c0 + t) * qk_stride + 8 * jc) * EB);
      if (t + 1 < nv) r1 = Ld8<TI>::load(kg + ((c0 + t + 1) * qk_stride + 8 * jc) * EB);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        f16x2 pr = {r0[e], r1[e]};
        *reinterpret_cast<f16x2*>(&sm.kt[(8 * jc + e) * kTS + t]) = pr;
      }
      f16x8 v0 = {}, v1 = {};
      if (t < nv) v0 = Ld8<TI>::load(vg + ((c0 + t) * v_stride + 8 * jc) * EB);
      if (t + 1 < nv) v1 = Ld8<TI>::load(vg + ((c0 + t + 1) * v_stride + 8 * jc) * EB);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        f16x2 pr = {v0[e], v1[e]};
        *reinterpret_cast<f16x2*>(&sm.vt[(8 * jc + e) * kTS + t]) = pr;
      }
    }
    if (w == 0) {
      const bool ok = l < nv;
      const size_t gi = static_cast<size_t>(c0 + l) * a.h_v + h;
      float gl = 0.0f, be = 0.0f;
      if (ok) {
        const float al = a.alpha[gi];
        gl = a.alpha_is_log ? al : __logf(al);
        gl = fmaxf(gl, -64.0f);
        be = a.beta ? a.beta[gi] : 1.0f;
      }
      // inclusive prefix sum of the log-decays over the 64 lanes
#pragma unroll
      for (int off = 1; off < kWave; off <<= 1) {
        const float y = __shfl_up(gl, off, kWave);
        if (l >= off) gl += y;
      }
      const float gC = __shfl(gl, kWave - 1, kWave);
      const float e_g = __expf(gl);
      sm.gcum[l] = gl;
      sm.gam[l] = e_g;
      sm.dec[l] = __expf(gC - gl);
      sm.beta[l] = be;
      sm.bg[l] = be * e_g;
    }
    __syncthreads();

    // ---- A = strict lower part of b_t e^{G_t-G_j} K K^T (fp32) ------------
    if (ERASE) {
      for (int job = w; job < 10; job += 4) {
        // lower-triangular 16x16 tiles in row-major order
        const int tr = job < 1 ? 0 : job < 3 ? 1 : job < 6 ? 2 : 3;
        const int tc = job - tr * (tr + 1) / 2;
        const int ta = 16 * tr + lr, tb_ = 16 * tc + lr;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < NKJ; ++ks) {
          f16x8 av = {}, bv = {};
          if (ta < nv) av = Ld8<TI>::load(kg + ((c0 + ta) * qk_stride + 32 * ks + 8 * lg) * EB);
          if (tb_ < nv) bv = Ld8<TI>::load(kg + ((c0 + tb_) * qk_stride + 32 * ks + 8 * lg) * EB);
          acc = mfma16x16x32(av, bv, acc);
        }
        const int col = 16 * tc + lr;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = 16 * tr + 4 * lg + r;
          float val = 0.0f;
          if (row > col)
            val = sm.beta[row] * __expf(sm.gcum[row] - sm.gcum[col]) * acc[r];
          sm.aw.a[row * kAS + col] = val;
        }
      }
      __syncthreads();

      // ---- (I + A)^{-1}: 16x16 diagonal blocks by forward substitution --
      if (w == 0) {
        const int b = l / 16, c = l % 16;
        float x[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float acc = (r == c) ? 1.0f : 0.0f;
          const float* arow = &sm.aw.a[(16 * b + r) * kAS + 16 * b];
#pragma unroll
          for (int m = 0; m < r; ++m) acc = fmaf(-arow[m], x[m], acc);
          x[r] = acc;
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) sm.tt.tm[(16 * b + r) * kAS + 16 * b + c] = x[r];
      }
      __syncthreads();
      // ---- off-diagonal blocks, one block column per wave ---------------
      // T_ij = -T_ii * sum_{m=j}^{i-1} A_im T_mj
#pragma unroll
      for (int s = 0; s < 3; ++s) {
        const int jb = w;
        const int ib = w + 1 + s;
        const bool act = ib <= 3;
        const int r = l / 4, c4 = 4 * (l % 4);
        if (act) {
          f32x4 x4 = {0.f, 0.f, 0.f, 0.f};
          for (int m = jb; m < ib; ++m) {
            const float* arow = &sm.aw.a[(16 * ib + r) * kAS + 16 * m];
#pragma unroll
            for (int mm = 0; mm < 16; ++mm) {
              const f32x4 tv = *reinterpret_cast<const f32x4*>(
                  &sm.tt.tm[(16 * m + mm) * kAS + 16 * jb + c4]);
              x4 += arow[mm] * tv;
            }
          }
          *reinterpret_cast<f32x4*>(&sm.tt.tm[(16 * ib + r) * kAS + 16 * jb + c4]) = x4;
        }
        __syncthreads();
        if (act) {
          f32x4 y4 = {0.f, 0.f, 0.f, 0.f};
          const float* trow = &sm.tt.tm[(16 * ib + r) * kAS + 16 * ib];
#pragma unroll
          for (int mm = 0; mm < 16; ++mm) {
            const f32x4 xv = *reinterpret_cast<const f32x4*>(
                &sm.tt.tm[(16 * ib + mm) * kAS + 16 * jb + c4]);
            y4 += trow[mm] * xv;
          }
          *reinterpret_cast<f32x4*>(&sm.tt.tm[(16 * ib + r) * kAS + 16 * jb + c4]) = -y4;
        }
        __syncthreads();
      }
      // ---- Tm diag(b) and Tm diag(b e^G) as fp16 ------------------------
      {
        float tv[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int idx = tid + kThreads * e;
          const int row = idx / kC, col = idx % kC;
          tv[e] = col <= row ? sm.tt.tm[row * kAS + col] : 0.0f;
        }
        __syncthreads();
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int idx = tid + kThreads * e;
          const int row = idx / kC, col = idx % kC;
          sm.tt.t16.tb[row * kTS + col] = static_cast<_Float16>(tv[e] * sm.beta[col]);
          sm.tt.t16.tbg[row * kTS + col] = static_cast<_Float16>(tv[e] * sm.bg[col]);
        }
      }
      __syncthreads();
    }

    // ---- U~ (erase) or U (erase-free) for this wave's value columns -------
    f32x4 U[4][NIT];
    if (ERASE) {
#pragma unroll
      for (int tt = 0; tt < 4; ++tt)
#pragma unroll
        for (int it = 0; it < NIT; ++it) {
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
          const int i = w * IW + 16 * it + lr;
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) {
            if (32 * ks > 16 * tt + 15) continue;  // Tm is lower triangular
            const f16x8 av = lds8(&sm.tt.t16.tb[(16 * tt + lr) * kTS + 32 * ks + 8 * lg]);
            const f16x8 bv = lds8(&sm.vt[i * kTS + 32 * ks + 8 * lg]);
            acc = mfma16x16x32(av, bv, acc);
          }
          U[tt][it] = acc;
        }
      // -W^T = -(K^T (Tm diag(b e^G))^T) for this wave's key columns, to LDS
      // as -W [t][j]
#pragma unroll
      for (int jt = 0; jt < NIT; ++jt)
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
          const int j = w * IW + 16 * jt + lr;
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) {
            if (32 * ks > 16 * tt + 15) continue;
            const f16x8 av = lds8(&sm.kt[j * kTS + 32 * ks + 8 * lg]);
            const f16x8 bv = lds8(&sm.tt.t16.tbg[(16 * tt + lr) * kTS + 32 * ks + 8 * lg]);
            acc = mfma16x16x32(av, bv, acc);
          }
          // acc: column t = 16tt + lr, rows j = w*IW + 16jt + 4lg + r
          const int t = 16 * tt + lr;
          *reinterpret_cast<f16x4*>(&sm.aw.w[t * kWS + w * IW + 16 * jt + 4 * lg]) =
              to_f16x4(-acc);
        }
    } else {
#pragma unroll
      for (int tt = 0; tt < 4; ++tt)
#pragma unroll
        for (int it = 0; it < NIT; ++it) {
          const int i = w * IW + 16 * it + lr;
          const f16x4 vv = lds4(&sm.vt[i * kTS + 16 * tt + 4 * lg]);
#pragma unroll
          for (int r = 0; r < 4; ++r)
            U[tt][it][r] = static_cast<float>(vv[r]) * sm.beta[16 * tt + 4 * lg + r];
        }
    }

    __syncthreads();  // -W complete; Tm tiles dead

    // ---- P o (Q K^T) into LDS (only the tiles the output product reads) ---
    if (want_o) {
      for (int job = w; job < 10; job += 4) {
        const int tr = job < 1 ? 0 : job < 3 ? 1 : job < 6 ? 2 : 3;
        const int tc = job - tr * (tr + 1) / 2;
        const int ta = 16 * tr + lr, tb_ = 16 * tc + lr;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < NKJ; ++ks) {
          f16x8 av = {}, bv = {};
          if (ta < nv) av = Ld8<TI>::load(qg + ((c0 + ta) * qk_stride + 32 * ks + 8 * lg) * EB);
          if (tb_ < nv) bv = Ld8<TI>::load(kg + ((c0 + tb_) * qk_stride + 32 * ks + 8 * lg) * EB);
          acc = mfma16x16x32(av, bv, acc);
        }
        const int col = 16 * tc + lr;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = 16 * tr + 4 * lg + r;
          float val = 0.0f;
          if (row >= col) val = __expf(sm.gcum[row] - sm.gcum[col]) * acc[r];
          sm.tt.pqk[row * kTS + col] = static_cast<_Float16>(val);
        }
      }
      // upper tiles (0,1) and (2,3) are read by the K = 32 steps below
      if (w == 0) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int idx = l + kWave * e;  // 0..255 over a 16x16 tile
          const int rr = idx / 16, cc = idx % 16;
          sm.tt.pqk[rr * kTS + 16 + cc] = static_cast<_Float16>(0.0f);
          sm.tt.pqk[(32 + rr) * kTS + 48 + cc] = static_cast<_Float16>(0.0f);
        }
      }
    }

    // ---- U = U~ - W S^T and O = Q S^T, one key k-step at a time ----------
    // S^T tiles 2kk and 2kk+1 form the fp16 B operand of k-step kk.
    f32x4 O[4][NIT];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
      for (int it = 0; it < NIT; ++it) O[tt][it] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (ERASE || want_o) {
#pragma unroll
      for (int kk = 0; kk < NKJ; ++kk) {
        f16x8 s16[NIT];
#pragma unroll
        for (int it = 0; it < NIT; ++it) s16[it] = to_f16x8(S[2 * kk][it], S[2 * kk + 1][it]);
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
          const int t = 16 * tt + lr;
          if (ERASE) {
            const f16x8 av = lds_perm(&sm.aw.w[t * kWS + 32 * kk], lg);
#pragma unroll
            for (int it = 0; it < NIT; ++it) U[tt][it] = mfma16x16x32(av, s16[it], U[tt][it]);
          }
          if (want_o) {
            f16x8 qa = {};
            if (t < nv) {
              const char* qrow = qg + ((c0 + t) * qk_stride + 32 * kk) * EB;
              qa = cat44(ld4_f16<TI>(qrow + 4 * lg * EB), ld4_f16<TI>(qrow + (16 + 4 * lg) * EB));
            }
#pragma unroll
            for (int it = 0; it < NIT; ++it) O[tt][it] = mfma16x16x32(qa, s16[it], O[tt][it]);
          }
        }
      }
    }

    if (want_o) {
      __syncthreads();  // P o QK^T complete
      // O = diag(e^G) Q S^T + (P o Q K^T) U
      f16x8 U16[2][NIT];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int it = 0; it < NIT; ++it) U16[ks][it] = to_f16x8(U[2 * ks][it], U[2 * ks + 1][it]);
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        const int t = 16 * tt + lr;
#pragma unroll
        for (int it = 0; it < NIT; ++it)
#pragma unroll
          for (int r = 0; r < 4; ++r) O[tt][it][r] *= sm.gam[16 * tt + 4 * lg + r];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          if (32 * ks > 16 * tt + 15) continue;
          const f16x8 av = lds_perm(&sm.tt.pqk[t * kTS + 32 * ks], lg);
#pragma unroll
          for (int it = 0; it < NIT; ++it) O[tt][it] = mfma16x16x32(av, U16[ks][it], O[tt][it]);
        }
#pragma unroll
        for (int it = 0; it < NIT; ++it)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int row = 16 * tt + 4 * lg + r;
            if (row < nv)
              store1<TO>(a.o, (static_cast<size_t>(c0 + row) * a.h_v + h) * D + w * IW + 16 * it + lr,
                         a.scale * O[tt][it][r]);
          }
      }
    }

    // ---- S^T <- e^{G_C} S^T + K^T diag(e^{G_C-G}) U -----------------------
    {
      f16x8 UD[2][NIT];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int it = 0; it < NIT; ++it) {
          f32x4 lo = U[2 * ks][it], hi = U[2 * ks + 1][it];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            lo[r] *= sm.dec[32 * ks + 4 * lg + r];
            hi[r] *= sm.dec[32 * ks + 16 + 4 * lg + r];
          }
          UD[ks][it] = to_f16x8(lo, hi);
        }
      const float gC = sm.gam[kC - 1];
#pragma unroll
      for (int jt = 0; jt < NJT; ++jt) {
        const _Float16* krow = &sm.kt[(16 * jt + lr) * kTS];
#pragma unroll
        for (int it = 0; it < NIT; ++it) S[jt][it] *= gC;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const f16x8 av = lds_perm(krow + 32 * ks, lg);
#pragma unroll
          for (int it = 0; it < NIT; ++it) S[jt][it] = mfma16x16x32(av, UD[ks][it], S[jt][it]);
        }
      }
    }
    __syncthreads();  // LDS reused by the next chunk
  }

#pragma unroll
  for (int jt = 0; jt < NJT; ++jt)
#pragma unroll
    for (int it = 0; it < NIT; ++it)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int j = 16 * jt + 4 * lg + r;
        const int i = w * IW + 16 * it + lr;
        a.s_out[sbase + static_cast<size_t>(j) * D + i] = S[jt][it][r];
      }
}

template <int D, typename TI, typename TO>
hipError_t launch3(const GdnArgs& a, hipStream_t s) {
  dim3 grid(a.n_seqs * a.h_v), block(kThreads);
  if (a.erase)
    hipLaunchKernelGGL((gdn_chunk_kernel<D, TI, TO, true>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((gdn_chunk_kernel<D, TI, TO, false>), grid, block, 0, s, a);
  return hipGetLastError();
}

template <int D, typename TI>
hipError_t launch2(const GdnArgs& a, hipStream_t s) {
  switch (a.dtype_o) {
    case SR_BF16: return launch3<D, TI, BF16>(a, s);
    case SR_F16: return launch3<D, TI, F16>(a, s);
    default: return launch3<D, TI, F32>(a, s);
  }
}

template <int D>
hipError_t launch1(const GdnArgs& a, hipStream_t s) {
  return a.dtype_qkv == SR_BF16 ? launch2<D, BF16>(a, s) : launch2<D, F16>(a, s);
}

}  // namespace

bool gdn_chunk_supports(int dtype_qkv, int d_k, int d_v) {
  return (dtype_qkv == SR_BF16 || dtype_qkv == SR_F16) && d_k == d_v &&
         (d_k == 64 || d_k == 128);
}

hipError_t launch_gdn_chunk(const GdnArgs& a, hipStream_t s) {
  if (a.n_seqs == 0) return hipSuccess;
  return a.d_k == 128 ? launch1<128>(a, s) : launch1<64>(a, s);
}

}  // namespace sr
