// Chunked gated-delta-rule replay on the gfx950 matrix cores.
//
// The per-token recurrence ("SuffixReplay", Eq. 4 with decay + rank-one
// erase; "Tail-Replay", section 2)
//     S_t = a_t S_{t-1} (I - b_t k_t k_t^T) + b_t v_t k_t^T,   o_t = S_t q_t
// is evaluated 64 tokens at a time.  Within a chunk (g_t = log a_t,
// G_t = sum_{s<=t} g_s; exact algebra of the recurrence):
//     A[t][j] = b_t e^{G_t-G_j} (k_t . k_j), j < t          (strictly lower)
//     (I + A) U = diag(b) (V - diag(e^G) K S^T)                (needs the carry)
//     O  = diag(e^G) Q S^T + (P o Q K^T) U,   P[t][j] = e^{G_t-G_j}, j <= t
//     S^T <- e^{G_C} S^T + K^T diag(e^{G_C-G}) U
// Erase-free mode (scalar decay only): A = 0, U = diag(b) V.
//
// The triangular system is solved by block forward substitution over 16-row
// blocks.  With A = diag(b) A~ (A~ without the b_t factor) and
// R~ = V - diag(e^G) K S^T, block row i reads
//     U_i = (I + A_ii)^{-1} diag(b_i) (R~_i - sum_{m<i} A~_im U_m):
// the four 16x16 diagonal blocks are inverted on the matrix cores at about
// fp32 accuracy (one wave each, see chunk_tiles) and stored with their
// columns scaled by b, the off-diagonal tiles hold -A~, so
// neither the right-hand side nor the off-diagonal tiles carry b; all
// products run on the matrix cores with register-resident operands.
// Solving for U directly (rather than for the S-independent pair
// T diag(b e^G) K, T diag(b) V and then combining them with S^T) keeps the
// solve to each wave's own value columns: no key-side columns, no
// intermediate tile in LDS and no barrier between the solve and the state
// products.
//
// Work layout: a workgroup holds HP value heads that share a key head, NW
// waves per head, and walks one sequence's chunks in order; it owns the
// value columns [c0, c0 + D/VS) of its heads (VS = 1, or 2 when a launch has
// too few chains to fill the CUs: value columns of S evolve independently,
// so the split is exact and only the key-side tiles are formed twice), and
// wave w of a head owns D/VS/NW of them (the launch picks HP, NW and VS from
// the number of (sequence, head) chains).  The transposed state S^T
// (d_k x d_v, fp32) stays in accumulator registers for the whole sequence.
// Accumulator tiles feed later products directly as operands: two
// vertically adjacent 16x16 tiles hold, per lane, the k-slots of a K = 32
// operand (see kkey), and the other operand is read from LDS in the same k
// order.  Operands are fp16 (bf16 inputs convert exactly); accumulation and
// the state are fp32.  The next chunk's K, Q and V are prefetched into
// registers while the current chunk computes, so each chunk has a single
// staging barrier.  Workgroups are numbered so that consecutive head groups
// of a sequence run on the same XCD (with one head per workgroup, the value
// heads sharing a key head then read K and Q through one L2).
#include "sr_common.hpp"
#include "sr_internal.hpp"

namespace sr {

namespace {

constexpr int kC = 64;         // chunk length (tokens)
// A workgroup holds HP value heads that share one key head, with NW waves
// per head (HP x NW = 4 or 8 waves), plus 4 producer waves in the
// producer/consumer form (PC), which stage the next chunk and form its
// tiles while the NW consumer waves run the current one:
//  * HP = 2, NW = 4 where the value heads per key head are even and there
//    are at least two (sequence, head) chains per CU: K and Q rows are
//    loaded and staged once and the raw K K^T / Q K^T tiles formed once for
//    both heads; one workgroup of 8 waves per CU;
//  * HP = 1, NW = 8, PC for at most one chain per CU: 16 value columns per
//    consumer wave, 12 waves (three per SIMD);
//  * HP = 1, NW = 4, VS = 2, PC for at most half a chain per CU: two
//    workgroups per chain, 16 value columns per consumer wave;
//  * HP = 1, NW = 4 otherwise: two workgroups of 4 waves per CU.
constexpr int kAS = kC + 8;    // fp16 row stride of -A
constexpr int kPS = kC + 8;    // fp16 row stride of P o QK^T
constexpr int kXcd = 8;        // XCDs; workgroups are dealt round-robin
// s_waitcnt immediate for vmcnt(0) with the other counters unconstrained
// (gfx9 encoding: vmcnt [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8])
constexpr int kWaitVmcnt0 = 0x0F70;
// State exponent.  Each wave keeps its columns of the state as S = 2^E S_reg
// (E >= 0, wave-uniform) and its U and outputs in the same units, so that
// the fp16 copies of S_reg and U stay far inside fp16's range (65504) for a
// state of any fp32 magnitude.  At every chunk start the wave checks
// max |S_reg|: above kSHi, or below kSLo while E > 0, it rescales S_reg by a
// power of two (exact) so the maximum lands just under 2^kSTarget.  States of
// ordinary size keep E = 0, where the arithmetic is the unscaled one.
constexpr float kSHi = 256.0f;
constexpr float kSLo = 8.0f;
constexpr int kSTarget = 7;

template <int D, int HP>
struct ChunkSmem {
  // Row strides (fp16 elements), chosen for LDS bank conflicts (32 banks of
  // 4 bytes, one 128-byte phase per cycle).  Q and V: 8 elements of padding,
  // so 16-byte row reads of 8 consecutive rows, and V's transpose reads, hit
  // distinct banks or at most 2-way.  K: 16 elements of padding plus a
  // swizzle (kswz: rows 4..7 of every 8 exchange their 16-byte column chunks
  // pairwise), so both its 16-byte row reads and its transpose reads are
  // conflict-free or 2-way; with a plain 8-element pad the transpose reads
  // would be 4-way under the state's key order (see kkey).
  static constexpr int kKS = D + 16;  // K rows
  static constexpr int kQS = D + 8;   // Q rows
  static constexpr int kWS = D + 8;   // V rows
  // Order: everything read with compile-time offsets lies below 64 KB, so a
  // DS instruction's 16-bit offset field holds the array start and one base
  // register serves many reads; K (last) is read through opaque per-lane
  // bases.  Every array starts on a 256-byte boundary (bank-neutral).
  // Per value head ([HP]): gates, inverse blocks, tiles and V; K and Q are
  // shared by the heads of the workgroup.
  float gcum[HP][kC];                // G_t log2(e) (base-2 exponent units)
  float gam[HP][kC];                 // e^{G_t}
  float dec[HP][kC];                 // e^{G_C - G_t}
  float beta[HP][kC];                // b_t (0 past the end of the sequence)
  _Float16 td[HP][4 * 16 * 16];      // (I + A_bb)^{-1} diag(b), row-major per block
  _Float16 a[HP][kC * kAS];          // -A~ (strictly lower off-diagonal blocks)
  _Float16 pqk[HP][kC * kPS];        // scale * P o (Q K^T)
  _Float16 q[kC * kQS];              // Q rows
  uint16_t w[HP][kC * kWS];          // raw V rows (input bits)
  _Float16 k[kC * kKS];              // K rows
};

// Storage position of column c in tiles that are read only as K = 32 MFMA
// operands (-A and P o QK^T): a K = 32 operand gives lane group g the
// k-slots {4g..4g+3, 16+4g..16+4g+3} of each 32-column group, which this
// order stores next to each other, so one 16-byte read fetches them.
__device__ __forceinline__ constexpr int kperm(int c) {
  return (c & ~31) + 8 * ((c & 15) >> 2) + 4 * ((c & 31) >> 4) + (c & 3);
}

// Four consecutive columns 4m..4m+3 land on four consecutive, 8-byte aligned
// storage positions (the tile epilogue stores them with one 8-byte write).
__device__ __forceinline__ constexpr bool kperm_quads_contiguous() {
  for (int c = 0; c < kC; c += 4)
    for (int r = 0; r < 4; ++r)
      if (kperm(c + r) != kperm(c) + r || kperm(c) % 4 != 0) return false;
  return kAS % 4 == 0 && kPS % 4 == 0;
}
static_assert(kperm_quads_contiguous(), "tile stores need column quads contiguous");

// Column swizzle of K row t (fp16 elements, XORed into the column): rows
// 4..7 of every 8 exchange their 16-byte column chunks pairwise.
__device__ __forceinline__ int kswz(int t) { return 8 * ((t >> 2) & 1); }

// Key held by element r of lane group g in state tile jt (rows of S^T).  The
// state's key order is chosen so that the 8 k-slots of lane group g in a
// K = 32 operand made of tiles 2m and 2m+1 are the 8 consecutive keys
// 32m + 8g .. 32m + 8g + 7: the K rows (right-hand side) and Q rows (outputs)
// that meet the state in a product are then one 16-byte read per lane.
__device__ __forceinline__ constexpr int kkey(int jt, int g, int r) {
  return 32 * (jt >> 1) + 8 * g + 4 * (jt & 1) + r;
}

// element (t, j) of the padded K and Q row tiles
template <int D>
__device__ __forceinline__ int kidx(int t, int j) {
  return t * ChunkSmem<D, 1>::kKS + j;
}
template <int D>
__device__ __forceinline__ int qidx(int t, int j) {
  return t * ChunkSmem<D, 1>::kQS + j;
}

__device__ __forceinline__ f16x8 lds8(const _Float16* p) {
  return *reinterpret_cast<const f16x8*>(p);
}
__device__ __forceinline__ f16x4 lds4(const _Float16* p) {
  return *reinterpret_cast<const f16x4*>(p);
}

// LDS transpose read (gfx950 ds_read_b64_tr_b16).  Within each group of 16
// lanes, lane m names 4 consecutive 16-bit elements that form row m/4, columns
// 4(m%4)..4(m%4)+3 of a 4 x 16 block, and receives column m of that block
// (rows 0..3).  For a row-major matrix with row stride S, lane l of the wave
// therefore passes  base + (l/4)*S + 4*(l%4)  to read rows R0+4(l/16)..+3 at
// column C0 + l%16, where base points at (R0, C0).
//
// Every transpose read of a tile goes through one base address that comes
// out of an opaque copy (tr_base), so the compiler keeps it in a single
// register instead of rematerialising it per read, and stays live until after
// the last read (tr_keep); the offset argument is a compile-time constant
// after unrolling and folds into the instruction.
__device__ __forceinline__ uint32_t tr_base(uint32_t lds_byte_addr) {
  uint32_t b;
  asm volatile("" : "=v"(b) : "0"(lds_byte_addr));
  return b;
}
__device__ __forceinline__ void tr_keep(uint32_t base) { asm volatile("" ::"v"(base)); }
__device__ __forceinline__ u16x4 lds_tr4(uint32_t base, int byte_off) {
  typedef __attribute__((__vector_size__(4 * sizeof(__fp16)))) __fp16 hx4;
  const auto lp = (__attribute__((address_space(3))) hx4*)(static_cast<uintptr_t>(base + byte_off));
  return __builtin_bit_cast(u16x4, __builtin_amdgcn_ds_read_tr16_b64_v4f16(lp));
}
// LDS byte address of a shared-memory object.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) char*)(p)));
}
__device__ __forceinline__ f16x4 as_f16x4(u16x4 v) { return __builtin_bit_cast(f16x4, v); }
// 16-byte LDS store at a byte address.
__device__ __forceinline__ void lds_store16(uint32_t addr, u16x8 v) {
  *(__attribute__((address_space(3))) u16x8*)(static_cast<uintptr_t>(addr)) = v;
}
// 16-byte LDS read at an opaque base plus a compile-time byte offset.
__device__ __forceinline__ f16x8 lds8_at(uint32_t base, int byte_off) {
  return *(const __attribute__((address_space(3))) f16x8*)(static_cast<uintptr_t>(base + byte_off));
}

__device__ __forceinline__ f32x4 mfma16x16x16(f16x4 a, f16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}

// Keeps the scheduler from hoisting the loads of later unrolled iterations
// above this point (which would make their registers live all at once).
#define SR_SCHED_FENCE() __builtin_amdgcn_sched_barrier(0)

// Raw 16-bit input rows -> fp16 (bf16 -> fp16 is exact in fp16's normal
// range); two elements per conversion instruction.
template <typename TI>
__device__ __forceinline__ u16x8 raw_to_f16x8(u16x8 v);
template <>
__device__ __forceinline__ u16x8 raw_to_f16x8<BF16>(u16x8 v) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 w = __builtin_bit_cast(u32x4, v);
  u32x4 o;
#pragma unroll
  for (int x = 0; x < 4; ++x) {
    const f16x2 h = {static_cast<_Float16>(__uint_as_float(w[x] << 16)),
                     static_cast<_Float16>(__uint_as_float(w[x] & 0xffff0000u))};
    o[x] = __builtin_bit_cast(uint32_t, h);
  }
  return __builtin_bit_cast(u16x8, o);
}
template <>
__device__ __forceinline__ u16x8 raw_to_f16x8<F16>(u16x8 v) {
  return v;
}
// One raw 16-bit input element -> fp32.
template <typename TI>
__device__ __forceinline__ float raw_to_f32(uint16_t b);
template <>
__device__ __forceinline__ float raw_to_f32<BF16>(uint16_t b) {
  return bf16_to_f32(b);
}
template <>
__device__ __forceinline__ float raw_to_f32<F16>(uint16_t b) {
  return static_cast<float>(__builtin_bit_cast(_Float16, b));
}

// fp32 tile as fp16 hi + lo parts (x - hi is exact in fp32), for products
// at about fp32 accuracy on the fp16 matrix cores.  The residual is written
// as an FMA with fp16 and fp32 operands rounded once to fp16, which is one
// mixed-precision instruction per element.
struct SplitF16 {
  f16x4 h, l;
};
__device__ __forceinline__ SplitF16 split_f16(f32x4 x) {
  SplitF16 s;
  float m1 = -1.0f;  // opaque, so the FMA is not folded into a subtraction
  asm("" : "+v"(m1));
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    s.h[r] = static_cast<_Float16>(x[r]);
    s.l[r] = static_cast<_Float16>(__builtin_fmaf(static_cast<float>(s.h[r]), m1, x[r]));
  }
  return s;
}
// a^T b + c for tiles a, b in the 16x16 accumulator layout (hi*hi + hi*lo +
// lo*hi, small terms first)
__device__ __forceinline__ f32x4 mfma_split(const SplitF16& a, const SplitF16& b, f32x4 c) {
  c = mfma16x16x16(a.l, b.h, c);
  c = mfma16x16x16(a.h, b.l, c);
  return mfma16x16x16(a.h, b.h, c);
}

// Tile jobs of wave W for one chunk.  Waves 0..3 of each head form the
// diagonal blocks A_bb (erase mode; b = the wave within the head) and invert
// I + A_bb.  The 16 other tiles are shared jobs: with 4 waves, wave W takes
// jobs W, W+4, W+8, W+12; with 8 waves, jobs 2W and 2W+1, each written once
// per head of the workgroup (the raw product is the same, the gate factors
// differ).  The job list is fixed at compile time so the whole section is
// straight-line code with immediate LDS offsets, and the k-steps of all jobs
// interleave.
//   A tile jobs:        (1,0) (2,0) (2,1) (3,0) (3,1) (3,2)
//   P o QK^T tile jobs: (0,0) (1,0) (1,1) (2,0) (2,1) (2,2) (3,0) (3,1) (3,2) (3,3)
template <int D, int HP, int NW, bool ERASE, bool WANT_O, int W>
__device__ __forceinline__ void chunk_tiles(ChunkSmem<D, HP>& sm, int lr, int lg, float scale) {
  constexpr int NKJ = D / 32;
  constexpr int kJob[16][3] = {{1, 1, 0}, {1, 2, 0}, {1, 2, 1}, {1, 3, 0}, {1, 3, 1}, {1, 3, 2},
                               {0, 0, 0}, {0, 1, 0}, {0, 1, 1}, {0, 2, 0}, {0, 2, 1}, {0, 2, 2},
                               {0, 3, 0}, {0, 3, 1}, {0, 3, 2}, {0, 3, 3}};
  constexpr int NWT = NW * HP;    // waves of the workgroup (4 or 8)
  constexpr int HW = W / NW;      // this wave's head
  constexpr int WQ = W % NW;      // its diagonal block (waves 0..3 of a head)
  constexpr bool kDiag = ERASE && WQ < 4;
  constexpr int NS = NWT == 4 ? 5 : 3;  // slot 0: diagonal block; then the jobs
  auto job = [](int q) constexpr { return NWT == 4 ? W + 4 * (q - 1) : 2 * W + (q - 1); };
  auto slot_on = [job](int q) constexpr {
    if (q == 0) return kDiag;
    return kJob[job(q)][0] == 1 ? ERASE : WANT_O;
  };
  auto slot_kk = [job](int q) constexpr { return q == 0 || kJob[job(q)][0] == 1; };
  auto slot_tr = [job](int q) constexpr { return q == 0 ? WQ : kJob[job(q)][1]; };
  auto slot_tc = [job](int q) constexpr { return q == 0 ? WQ : kJob[job(q)][2]; };
  auto slot_h0 = [](int q) constexpr { return q == 0 ? HW : 0; };   // first head written
  auto slot_nh = [](int q) constexpr { return q == 0 ? 1 : HP; };   // heads written
  f32x4 acc[NS];
#pragma unroll
  for (int q = 0; q < NS; ++q) acc[q] = f32x4{0.f, 0.f, 0.f, 0.f};
  // Element layout: the diagonal block (slot 0) stays in the accumulator
  // layout the inverse works in (lane (lr, lg) holds rows 16tr+4lg+r of column
  // 16tc+lr).  The other tiles are formed transposed (operands swapped, the
  // same products), so lane (lr, lg) holds row 16tr+lr at the 4 consecutive
  // columns 16tc+4lg+r, which sit next to each other in the kperm storage
  // order: one 8-byte LDS store per tile and head.
  auto el_row = [=](int q, int r) { return q == 0 ? 16 * slot_tr(q) + 4 * lg + r : 16 * slot_tr(q) + lr; };
  auto el_col = [=](int q, int r) { return q == 0 ? 16 * slot_tc(q) + lr : 16 * slot_tc(q) + 4 * lg + r; };
  // decay / gate factors of this lane's tile elements, formed before the
  // products (they do not depend on them): masked b_t e^{G_t-G_j} for the
  // diagonal A block, -e^{G_t-G_j} for the others (-A~), scale e^{G_t-G_j}
  // for P o QK^T.  The gate values are read unconditionally (four rows or
  // columns per vector read) and the causal mask applied by selects, so no
  // LDS read sits behind a branch.
  float f[NS][HP][4];
#pragma unroll
  for (int q = 0; q < NS; ++q) {
    if (!slot_on(q)) continue;
#pragma unroll
    for (int hh = 0; hh < slot_nh(q); ++hh) {
      const int hd = slot_h0(q) + hh;
      // the lane's scalar (column for slot 0, row otherwise) and its 4-vector
      const float g1 = sm.gcum[hd][q == 0 ? el_col(q, 0) : el_row(q, 0)];
      const f32x4 g4 = *reinterpret_cast<const f32x4*>(&sm.gcum[hd][q == 0 ? el_row(q, 0) : el_col(q, 0)]);
      // b_t only on the diagonal block (the inverse needs the true A_bb); the
      // off-diagonal A tiles hold -A~, the P o QK^T tiles carry the scale
      const f32x4 wrow = q == 0 ? *reinterpret_cast<const f32x4*>(&sm.beta[hd][el_row(q, 0)])
                         : slot_kk(q) ? f32x4{1.0f, 1.0f, 1.0f, 1.0f}
                                      : f32x4{scale, scale, scale, scale};
      const float sgn = (q == 0 || !slot_kk(q)) ? 1.0f : -1.0f;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = el_row(q, r), col = el_col(q, r);
        const float gd = q == 0 ? g4[r] - g1 : g1 - g4[r];  // G_row - G_col
        const float v = sgn * wrow[r] * __builtin_amdgcn_exp2f(gd);
        const bool keep = slot_kk(q) ? row > col : row >= col;
        f[q][hh][r] = keep ? v : 0.0f;
      }
    }
  }
  // this lane's row lr, k-slots 8lg.. of the K and Q tiles
  // (tile row offsets are multiples of 16, so K's swizzle depends on lr only)
  const uint32_t kl = tr_base(lds_addr(&sm.k[kidx<D>(lr, (8 * lg) ^ kswz(lr))]));
  const uint32_t ql = WANT_O ? tr_base(lds_addr(&sm.q[qidx<D>(lr, 8 * lg)])) : 0u;
#pragma unroll
  for (int ks = 0; ks < NKJ; ++ks) {
#pragma unroll
    for (int q = 0; q < NS; ++q) {
      if (!slot_on(q)) continue;
      const f16x8 av = slot_kk(q) ? lds8_at(kl, 2 * kidx<D>(16 * slot_tr(q), 32 * ks))
                                  : lds8_at(ql, 2 * qidx<D>(16 * slot_tr(q), 32 * ks));
      const f16x8 bv = lds8_at(kl, 2 * kidx<D>(16 * slot_tc(q), 32 * ks));
      acc[q] = q == 0 ? mfma16x16x32(av, bv, acc[q]) : mfma16x16x32(bv, av, acc[q]);
    }
  }
  tr_keep(kl);
  if (WANT_O) tr_keep(ql);
  // epilogues: masked, decay-weighted tiles to LDS (the diagonal A block
  // stays in registers for the inverse)
  f32x4 nd = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int q = 0; q < NS; ++q) {
    if (!slot_on(q)) continue;
#pragma unroll
    for (int hh = 0; hh < slot_nh(q); ++hh) {
      const int hd = slot_h0(q) + hh;
      if (q == 0) {
#pragma unroll
        for (int r = 0; r < 4; ++r) nd[r] = f[q][hh][r] * acc[q][r];
      } else {
        f16x4 o;
#pragma unroll
        for (int r = 0; r < 4; ++r) o[r] = static_cast<_Float16>(f[q][hh][r] * acc[q][r]);
        _Float16* dst = slot_kk(q) ? &sm.a[hd][el_row(q, 0) * kAS + kperm(el_col(q, 0))]
                                   : &sm.pqk[hd][el_row(q, 0) * kPS + kperm(el_col(q, 0))];
        *reinterpret_cast<f16x4*>(dst) = o;
      }
    }
  }
  if (kDiag) {
    // T = (I + N)^{-1} for this wave's diagonal block N = A_bb (strictly
    // lower, 16 x 16), on the matrix cores.  N is held in the accumulator
    // layout: lane (lr, lg) has N[4 lg + r][lr], r = 0..3.  Split N = D + L
    // into its 4 x 4 diagonal blocks D and the strictly block-lower rest L;
    // then I + N = (I + D)(I + M) with M = (I + D)^{-1} L, and since M is
    // strictly block-lower over 4 blocks (M^4 = 0)
    //     T = (I + M)^{-1} (I + D)^{-1},  (I + M)^{-T} = I - Z + Z^2 - Z^3,
    //     Z = M^T.
    // (I + D)^{-1} comes in closed form from the six entries of each 4 x 4
    // block, which sit in one quad of lanes (the quad whose columns meet the
    // lane group's rows) and are broadcast within it by DPP.  A product
    // mfma(a, b) of two operands held in the accumulator layout of X and Y
    // is X^T Y, so every operand below is an accumulator tile; each is split
    // into fp16 hi + lo parts (three MFMAs per product), which keeps the
    // result at fp32 accuracy before its one fp16 rounding.  The series has
    // only four terms of 4 x 4 block structure, so it does not cancel
    // catastrophically even for a block of identical keys.
    const int j = lr & 3;                    // column within the 4 x 4 block
    const bool dblk = (lr >> 2) == lg;       // the lane's rows meet its column's block
    const bool lblk = (lr >> 2) < lg;        // strictly block-lower position
    const float e10 = dpp_f32<0x00, 0xf>(nd[1]), e20 = dpp_f32<0x00, 0xf>(nd[2]);
    const float e30 = dpp_f32<0x00, 0xf>(nd[3]), e21 = dpp_f32<0x55, 0xf>(nd[2]);
    const float e31 = dpp_f32<0x55, 0xf>(nd[3]), e32 = dpp_f32<0xaa, 0xf>(nd[3]);
    // (I + D_blk)^{-1}, unit lower triangular: entries i_rj, r > j
    const float i10 = -e10, i21 = -e21, i32 = -e32;
    const float i20 = fmaf(e21, e10, -e20);
    const float i31 = fmaf(e32, e21, -e31);
    const float i30 = fmaf(-e32, i20, fmaf(-e31, i10, -e30));
    f32x4 di, dt, id, lm;  // (I + D)^{-1}, its transpose, I, L (accumulator layout)
    di[0] = j == 0 ? 1.0f : 0.0f;
    di[1] = j == 0 ? i10 : j == 1 ? 1.0f : 0.0f;
    di[2] = j == 0 ? i20 : j == 1 ? i21 : j == 2 ? 1.0f : 0.0f;
    di[3] = j == 0 ? i30 : j == 1 ? i31 : j == 2 ? i32 : 1.0f;
    dt[0] = j == 0 ? 1.0f : j == 1 ? i10 : j == 2 ? i20 : i30;
    dt[1] = j == 1 ? 1.0f : j == 2 ? i21 : j == 3 ? i31 : 0.0f;
    dt[2] = j == 2 ? 1.0f : j == 3 ? i32 : 0.0f;
    dt[3] = j == 3 ? 1.0f : 0.0f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      di[r] = dblk ? di[r] : 0.0f;
      dt[r] = dblk ? dt[r] : 0.0f;
      id[r] = dblk && j == r ? 1.0f : 0.0f;
      lm[r] = lblk ? nd[r] : 0.0f;
    }
    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
    const SplitF16 sl = split_f16(lm), sdt = split_f16(dt);
    const f32x4 m = mfma_split(sdt, sl, z);    // M = (I + D)^{-1} L
    const f32x4 mt = mfma_split(sl, sdt, z);   // M^T
    const SplitF16 snm = split_f16(-m);
    f32x4 x = id - mt;                         // I - Z
    x = mfma_split(snm, split_f16(x), id);     // I - Z (I - Z)
    x = mfma_split(snm, split_f16(x), id);     // (I + Z)^{-1}
    // T^T = (I + D)^{-T} (I + M)^{-T}: lane (lr, lg) gets T[lr][4 lg + r],
    // stored as (I + A_bb)^{-1} diag(b) (column 4 lg + r scaled by its b_t),
    // each value pinned in fp32 before its fp16 rounding so no template
    // instance fuses the scaling with the conversion
    const f32x4 tt = mfma_split(split_f16(di), split_f16(x), z);
    const f32x4 bc = *reinterpret_cast<const f32x4*>(&sm.beta[HW][16 * WQ + 4 * lg]);
    f16x4 o;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float v = tt[r] * bc[r];
      asm volatile("" : "+v"(v));
      o[r] = static_cast<_Float16>(v);
    }
    *reinterpret_cast<f16x4*>(&sm.td[HW][WQ * 256 + lr * 16 + 4 * lg]) = o;
  }
}

// PC: producer/consumer form (one head of NW consumer waves): 4 more waves
// per workgroup stage chunk c + 1 and form its tiles while the consumer
// waves run chunk c's state work, on two LDS buffers.
constexpr int kProducers = 4;  // producer waves of the PC form
// Launches that order their chains longest first: the plain forms (the
// producer/consumer forms run at most one chain per CU at a time) of 2 to
// kLptMax sequences (each workgroup ranks them all).
constexpr int kLptMax = 256;
template <bool PC>
__host__ __device__ constexpr bool lpt_launch(int n_seqs) {
  return !PC && n_seqs >= 2 && n_seqs <= kLptMax;
}
template <int D, typename TI, typename TO, bool ERASE, bool WANT_O, int HP, int NW, int VS, bool PC>
__global__ __launch_bounds__(64 * (NW * HP + (PC ? kProducers : 0)), NW * HP == 4 && !PC ? 2 : 1) void
gdn_chunk_kernel(GdnArgs a, int units_per_xcd) {
  static_assert(!PC || (HP == 1 && (NW == 4 || NW == 8)), "the producer/consumer form has one head");
  constexpr int kThreads = 64 * NW * HP;  // the (consumer) waves' threads
  // threads that load and stage the chunks: the producers in PC, else all
  constexpr int kLoaders = PC ? 64 * kProducers : kThreads;
  constexpr int DV = D / VS;      // value columns of the workgroup (per head)
  constexpr int IW = DV / NW;     // value columns per wave
  constexpr int NIT = IW / 16;    // 16-wide column tiles per wave
  constexpr int NJT = D / 16;     // 16-wide key tiles
  constexpr int NKJ = D / 32;     // K = 32 steps over the key dimension
  constexpr int CPR = D / 8;      // 16-byte chunks per row
  constexpr int NPF = kC * CPR / kLoaders;  // 16-byte K (and Q) row pieces per loader
  constexpr int VCPH = CPR / VS;            // 16-byte V pieces per token row and head
  constexpr int VCP = VCPH * HP;            // 16-byte V pieces per token row (all heads)
  constexpr int NPFV = kC * VCP / kLoaders; // V pieces per loader
  constexpr int kWS = ChunkSmem<D, HP>::kWS;
  static_assert(NIT >= 1 && IW % 16 == 0, "D too small");
  static_assert(kC * CPR % kLoaders == 0 && kLoaders % VCP == 0,
                "staging pieces must divide evenly");

  __shared__ ChunkSmem<D, HP> smb[PC ? 2 : 1];

  // XCD-aware numbering: consecutive (sequence, head group) units share an
  // XCD (with one head per workgroup, the value heads of a key head then
  // read K and Q through one L2).
  // (with VS > 1 the VS column slices of one chain are consecutive units, so
  // they share an XCD and read the chain's K and Q through one L2)
  const int groups = a.h_v / HP;  // head groups per sequence
  const int tid = threadIdx.x;
  int n, hgrp, slice;  // sequence, head group and column slice of the workgroup
  if (lpt_launch<PC>(a.n_seqs)) {
    // Longest chains first: every workgroup ranks the sequences by length
    // (descending, ties by index), and XCD x runs the sequences of ranks
    // x, x + 8, x + 16, ... in that order with all head groups of a
    // sequence in a row.  A ragged batch then does not end with a few long
    // chains on a few CUs; each chain's arithmetic is unchanged.
    __shared__ int lpt_len[kLptMax], lpt_seq[kLptMax];
    for (int e = tid; e < a.n_seqs; e += blockDim.x) lpt_len[e] = a.cu[e + 1] - a.cu[e];
    __syncthreads();
    for (int e = tid; e < a.n_seqs; e += blockDim.x) {
      const int le = lpt_len[e];
      int r = 0;
      for (int t = 0; t < a.n_seqs; ++t) {
        const int lt = lpt_len[t];
        r += (lt > le || (lt == le && t < e)) ? 1 : 0;
      }
      lpt_seq[r] = e;
    }
    __syncthreads();
    const int j = blockIdx.x / kXcd;
    const int rho = kXcd * (j / groups) + static_cast<int>(blockIdx.x % kXcd);
    if (rho >= a.n_seqs) return;  // padding workgroup
    n = lpt_seq[rho];
    hgrp = j % groups;
    slice = 0;
  } else {
    const int unit = (blockIdx.x % kXcd) * units_per_xcd + blockIdx.x / kXcd;
    if (unit >= a.n_seqs * groups * VS) return;  // padding workgroup
    n = unit / (groups * VS);
    hgrp = (unit / VS) % groups;
    slice = unit % VS;
  }
  const int hb = hgrp * HP;     // first value head of the workgroup
  const int col0 = slice * DV;  // first value column of the workgroup
  const int g = hb / (a.h_v / a.h_k);
  const int w = __builtin_amdgcn_readfirstlane(tid / kWave);  // wave-uniform
  const int hp = PC ? 0 : w / NW;  // this wave's head within the workgroup
  const int wq = w % NW;  // this wave within its head
  const int h = hb + hp;
  constexpr bool want_o = WANT_O;
  const size_t qk_row = static_cast<size_t>(a.h_k) * D;  // elements per token
  const size_t v_row = static_cast<size_t>(a.h_v) * D;
  const uint16_t* kg = static_cast<const uint16_t*>(a.k) + static_cast<size_t>(g) * D;
  const uint16_t* qg = want_o ? static_cast<const uint16_t*>(a.q) + static_cast<size_t>(g) * D
                              : nullptr;
  // V rows of the workgroup's heads (adjacent in each token row)
  const uint16_t* vg = static_cast<const uint16_t*>(a.v) + static_cast<size_t>(hb) * D + col0;

  // S^T accumulators: tile (jt, it) = 16 key rows, value columns
  // w*IW + 16it..; lane holds column lr and the keys kkey(jt, lg, 0..3).
  f32x4 S[NJT][NIT];
  int lr = tid % 16, lg = (tid / 16) % 4, l = tid % kWave;
  const size_t sbase = (static_cast<size_t>(n) * a.h_v + h) * D * D;
#pragma unroll
  for (int jt = 0; jt < NJT; ++jt)
#pragma unroll
    for (int it = 0; it < NIT; ++it)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int j = kkey(jt, lg, r);
        const int i = col0 + wq * IW + 16 * it + lr;
        S[jt][it][r] = a.s0 ? a.s0[sbase + static_cast<size_t>(j) * D + i] : 0.0f;
      }
  // Retire the initial-state loads here: otherwise the compiler's wait
  // insertion cannot tell at the loop's first read of S whether they are
  // done, and waits for every outstanding load there in each chunk (which
  // would include the next chunk's prefetch).
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);

  // P o QK^T tiles (0,1) and (2,3) are read as zeros by the K = 32 steps of
  // the output product and never written otherwise
  for (int b = 0; b < (PC ? 2 : 1); ++b)
    for (int e = tid; e < 256 * HP; e += kThreads) {
      const int hh = e / 256, rr = (e % 256) / 16, cc = e % 16;
      smb[b].pqk[hh][rr * kPS + kperm(16 + cc)] = static_cast<_Float16>(0.0f);
      smb[b].pqk[hh][(32 + rr) * kPS + kperm(48 + cc)] = static_cast<_Float16>(0.0f);
    }

  const int t_begin = a.cu[n];
  const int t_end = a.cu[n + 1];

  // ---- prefetch registers (raw input bits) for the next chunk -------------
  // Addresses are a uniform row base (scalar registers) plus a per-lane
  // offset that does not change between chunks.
  u16x8 pk[NPF], pq[NPF], pv[NPFV];
  float pa = 0.0f, pb = 0.0f;
  // this thread's 16-byte piece: row (w*64 + l) / CPR, column 8 * ((w*64 + l) % CPR)
  // (PC: the producer waves load, numbered from 0)
  const int lw = PC ? w - NW * HP : w;
  auto lane_row = [&]() { return (static_cast<unsigned>(lw) * kWave + static_cast<unsigned>(l)) / CPR; };
  auto lane_col = [&]() { return 8u * ((static_cast<unsigned>(lw) * kWave + static_cast<unsigned>(l)) % CPR); };
  // byte offsets from a uniform row base: 32-bit and unsigned, so the loads
  // take the scalar-base + vector-offset form without 64-bit address math
  auto kq_off = [&]() { return 2u * (lane_row() * static_cast<unsigned>(qk_row) + lane_col()); };
  // V: this thread's piece of a token row of all the workgroup's heads
  auto v_lane_row = [&]() { return (static_cast<unsigned>(lw) * kWave + static_cast<unsigned>(l)) / VCP; };
  auto v_lane_piece = [&]() { return (static_cast<unsigned>(lw) * kWave + static_cast<unsigned>(l)) % VCP; };
  auto v_off = [&]() {
    const unsigned cp = v_lane_piece();
    return 2u * (v_lane_row() * static_cast<unsigned>(v_row) + static_cast<unsigned>(D) * (cp / VCPH) +
                 8u * (cp % VCPH));
  };
  // One 16-byte piece e of the next chunk's K, Q or V rows per thread (zero
  // past the end of the sequence), and the next chunk's gates (wave 0).
  auto pf_k = [&](int e, int c0n) {
    const int row = static_cast<int>(lane_row()) + (kLoaders / CPR) * e;
    const uint16_t* kb = kg + static_cast<size_t>(c0n + (kLoaders / CPR) * e) * qk_row;
    pk[e] = u16x8{};
    if (row < t_end - c0n)
      pk[e] = *reinterpret_cast<const u16x8*>(reinterpret_cast<const char*>(kb) + kq_off());
  };
  auto pf_q = [&](int e, int c0n) {
    if (!want_o) return;
    const int row = static_cast<int>(lane_row()) + (kLoaders / CPR) * e;
    const uint16_t* qb = qg + static_cast<size_t>(c0n + (kLoaders / CPR) * e) * qk_row;
    pq[e] = u16x8{};
    if (row < t_end - c0n)
      pq[e] = *reinterpret_cast<const u16x8*>(reinterpret_cast<const char*>(qb) + kq_off());
  };
  auto pf_v = [&](int e, int c0n) {
    const int row = static_cast<int>(v_lane_row()) + (kLoaders / VCP) * e;
    const uint16_t* vb = vg + static_cast<size_t>(c0n + (kLoaders / VCP) * e) * v_row;
    pv[e] = u16x8{};
    if (row < t_end - c0n)
      pv[e] = *reinterpret_cast<const u16x8*>(reinterpret_cast<const char*>(vb) + v_off());
  };
  auto pf_gates = [&](int c0n) {
    if (wq == 0) {
      pa = 0.0f;
      pb = 0.0f;
      if (l < t_end - c0n) {
        const size_t g0 = static_cast<size_t>(c0n) * a.h_v + h;
        const unsigned go = 4u * static_cast<unsigned>(l) * static_cast<unsigned>(a.h_v);
        pa = *reinterpret_cast<const float*>(reinterpret_cast<const char*>(a.alpha + g0) + go);
        pb = a.beta ? *reinterpret_cast<const float*>(reinterpret_cast<const char*>(a.beta + g0) + go) : 1.0f;
      }
    }
  };
  // Load slot s of a chunk: K pieces, then Q pieces, then V pieces.  Inside
  // the chunk loop the slots are issued one or two at a time at fixed points
  // of the compute (the call sites are compile-time constants after
  // unrolling), so the CU's vector-memory path never sees all waves' loads
  // of a chunk at once: a wave whose load cannot be accepted stalls in
  // order, and a burst of 12 loads per wave cost ~2K cycles per chunk.
  constexpr int kSlots = 2 * NPF + NPFV;
  auto pf_slot = [&](int slot, int c0n) {
    if (slot < NPF) pf_k(slot, c0n);
    else if (slot < 2 * NPF) pf_q(slot - NPF, c0n);
    else pf_v(slot - 2 * NPF, c0n);
  };
  auto prefetch_all = [&](int c0n) {
    pf_gates(c0n);
#pragma unroll
    for (int slot = 0; slot < kSlots; ++slot) pf_slot(slot, c0n);
  };
  // Converts the prefetched raw K and Q to fp16 in place (V stays raw: it
  // only enters fp32 arithmetic) and scans the next
  // chunk's log-decays (wave 0, lane = token), once the loads have landed.
  float n_g = 0.0f, n_eg = 1.0f, n_dec = 1.0f, n_be = 0.0f;
  auto prepare = [&](int c0n) {
    const int nvn = min(kC, t_end - c0n);
#pragma unroll
    for (int e = 0; e < NPF; ++e) {
      pk[e] = raw_to_f16x8<TI>(pk[e]);
      if (want_o) pq[e] = raw_to_f16x8<TI>(pq[e]);
    }
    if (wq == 0) {
      float gl = 0.0f;
      if (l < nvn) {
        gl = a.alpha_is_log ? pa : __logf(pa);
        gl = fmaxf(gl, -64.0f);
      }
      n_be = l < nvn ? pb : 0.0f;
      gl = wave_inclusive_sum(gl);
      const float gC = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(gl), kWave - 1));
      n_g = gl * 1.4426950408889634f;  // base-2 units for the tile exponents
      n_eg = __expf(gl);
      n_dec = __expf(gC - gl);
    }
  };
  if (t_begin < t_end && (!PC || w >= NW * HP)) {
    prefetch_all(t_begin);
    prepare(t_begin);
  }
  int sexp = 0;  // state exponent E of this wave (S = 2^E S_reg)

  // ---- the pieces of one chunk ------------------------------------------
  // The plain launch runs them in order for each chunk with barriers in
  // between; the producer/consumer launch (PC) runs the staging and tiles of
  // chunk c + 1 (producer waves) beside the state work of chunk c (consumer
  // waves), on two LDS buffers.
  int tro = 0, trv = 0;  // this lane's transpose-read offsets in the K and V tiles
  // U accumulators: tile (tt, it) = token rows 16tt.., value columns
  // w*IW + 16it..
  f32x4 U[4][NIT];
  // fp16 copy of the state (B operand of K S^T, A operand of the outputs),
  // converted once per chunk
  f16x8 S16[NKJ][NIT];
  float s_dn = 1.0f, s_up = 1.0f;
  // the next chunk's loads are issued in slots spread over the compute: pfn
  // is the next slot, pf_c0 the chunk they load (none when !pf_more)
  int pfn = 0, pf_c0 = 0;
  bool pf_more = false;
  auto pf_next = [&](int n) {
#pragma unroll
    for (int i = 0; i < n; ++i) {
      if (pf_more && pfn < kSlots) pf_slot(pfn, pf_c0);
      ++pfn;
    }
  };
  auto coords = [&]() {
      // Re-derive the lane coordinates each chunk through an opaque copy so
      // that the many lane-dependent LDS/global addresses are recomputed in the
      // loop instead of being hoisted out of it (which would pin one register
      // per address for the whole sequence).
      {
        unsigned t_ = tid;
        asm volatile("" : "+v"(t_));
        l = t_ & (kWave - 1);
        lr = t_ & 15;
        lg = (t_ >> 4) & 3;
        // K transpose reads: token row (l >> 2) of a 16-row block, the 4 keys
        // kkey(jt, l & 3, 0..3) (8 (l & 3) + a per-tile constant), swizzled
        tro = (l >> 2) * ChunkSmem<D, HP>::kKS + ((8 * (l & 3)) ^ kswz(l >> 2));
        trv = (l >> 2) * kWS + 4 * (l & 3);
      }
  };
  auto stage = [&](ChunkSmem<D, HP>& sm) {
      // ---- stage this chunk: K, Q, V rows (already fp16) and gate scalars --
#pragma unroll
      for (int e = 0; e < NPF; ++e) {
        const unsigned row = lane_row() + (kLoaders / CPR) * e, col = lane_col();
        lds_store16(lds_addr(sm.k) + 2 * (row * ChunkSmem<D, HP>::kKS + (col ^ kswz(row))), pk[e]);
        if (want_o) lds_store16(lds_addr(sm.q) + 2 * (row * ChunkSmem<D, HP>::kQS + col), pq[e]);
      }
#pragma unroll
      for (int e = 0; e < NPFV; ++e) {
        const unsigned row = v_lane_row() + (kLoaders / VCP) * e, cp = v_lane_piece();
        lds_store16(lds_addr(&sm.w[cp / VCPH][0]) + 2 * (row * kWS + col0 + 8 * (cp % VCPH)), pv[e]);
      }
      if (wq == 0) {
        sm.gcum[hp][l] = n_g;
        sm.gam[hp][l] = n_eg;
        sm.dec[hp][l] = n_dec;
        sm.beta[hp][l] = n_be;
      }
  };
  auto tiles = [&](ChunkSmem<D, HP>& sm) {
      // ---- A (erase) and P o QK^T: lower-triangular 16x16 tiles -------------
      // Every wave forms the diagonal block of its head's rows 16 (w % 4)..
      // and inverts it (a wave-local LDS round trip, no barrier), and takes its
      // share of the off-diagonal A tiles and the P o QK^T tiles.
      if constexpr (PC) {
        // the producers split the tile jobs as a 4-wave workgroup would
        switch (w - NW * HP) {
          case 0: chunk_tiles<D, HP, kProducers, ERASE, WANT_O, 0>(sm, lr, lg, a.scale); break;
          case 1: chunk_tiles<D, HP, kProducers, ERASE, WANT_O, 1>(sm, lr, lg, a.scale); break;
          case 2: chunk_tiles<D, HP, kProducers, ERASE, WANT_O, 2>(sm, lr, lg, a.scale); break;
          default: chunk_tiles<D, HP, kProducers, ERASE, WANT_O, 3>(sm, lr, lg, a.scale); break;
        }
      } else {
        switch (w) {
          case 0: chunk_tiles<D, HP, NW, ERASE, WANT_O, 0>(sm, lr, lg, a.scale); break;
          case 1: chunk_tiles<D, HP, NW, ERASE, WANT_O, 1>(sm, lr, lg, a.scale); break;
          case 2: chunk_tiles<D, HP, NW, ERASE, WANT_O, 2>(sm, lr, lg, a.scale); break;
          case 3: chunk_tiles<D, HP, NW, ERASE, WANT_O, 3>(sm, lr, lg, a.scale); break;
          case 4: if constexpr (NW * HP == 8) chunk_tiles<D, HP, NW, ERASE, WANT_O, 4>(sm, lr, lg, a.scale); break;
          case 5: if constexpr (NW * HP == 8) chunk_tiles<D, HP, NW, ERASE, WANT_O, 5>(sm, lr, lg, a.scale); break;
          case 6: if constexpr (NW * HP == 8) chunk_tiles<D, HP, NW, ERASE, WANT_O, 6>(sm, lr, lg, a.scale); break;
          default: if constexpr (NW * HP == 8) chunk_tiles<D, HP, NW, ERASE, WANT_O, 7>(sm, lr, lg, a.scale); break;
        }
      }
  };
  auto part1 = [&](ChunkSmem<D, HP>& sm) {
      // ---- state exponent check (S = 2^E S_reg) -----------------------------
      {
        float m = 0.0f;
#pragma unroll
        for (int jt = 0; jt < NJT; ++jt)
#pragma unroll
          for (int it = 0; it < NIT; ++it)
#pragma unroll
            for (int r = 0; r < 4; ++r) m = fmaxf(m, fabsf(S[jt][it][r]));
        const bool over = __builtin_amdgcn_ballot_w64(m > kSHi) != 0;
        const bool under = sexp > 0 && __builtin_amdgcn_ballot_w64(m >= kSLo) == 0;
        if (over || under) {
          // rare: rescale S_reg so that its maximum lands just under 2^kSTarget
          const float mw = wave_max_nonneg(m);
          int e = 0;
          (void)frexpf(mw, &e);  // mw < 2^e
          int k = (mw > 0.0f && mw <= 3.0e38f) ? e - kSTarget : -sexp;
          k = max(k, -sexp);     // E stays >= 0
          k = min(k, 100);
          k = __builtin_amdgcn_readfirstlane(k);
          sexp += k;
          const float f = ldexpf(1.0f, -k);
#pragma unroll
          for (int jt = 0; jt < NJT; ++jt)
#pragma unroll
            for (int it = 0; it < NIT; ++it) S[jt][it] *= f;
        }
      }
      // 2^-E: applied to V (so U is in the state's units); 2^E: to the outputs
      s_dn = ldexpf(1.0f, -sexp);
      s_up = ldexpf(1.0f, sexp);

#pragma unroll
      for (int kk = 0; kk < NKJ; ++kk)
#pragma unroll
        for (int it = 0; it < NIT; ++it) S16[kk][it] = to_f16x8(S[2 * kk][it], S[2 * kk + 1][it]);
      // transpose-read base of this lane in the V tile at this wave's columns
      const uint32_t xv = tr_base(lds_addr(&sm.w[hp][0]) + 2 * (col0 + wq * IW + trv));
      if (ERASE) {
        // ---- right-hand side R~ = V - diag(e^G) K S^T ------------------------
        // K S^T for this wave's value columns, one key k-step at a time: S^T
        // tiles 2kk and 2kk+1 form the fp16 B operand of k-step kk, K rows the
        // A operand in the same k order.
#pragma unroll
        for (int tt = 0; tt < 4; ++tt)
#pragma unroll
          for (int it = 0; it < NIT; ++it) U[tt][it] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < NKJ; ++kk) {
          SR_SCHED_FENCE();
          pf_next(1);
#pragma unroll
          for (int tt = 0; tt < 4; ++tt) {
            const int t = 16 * tt + lr;
            const f16x8 kb = lds8(&sm.k[kidx<D>(t, (32 * kk + 8 * lg) ^ kswz(t))]);
#pragma unroll
            for (int it = 0; it < NIT; ++it) U[tt][it] = mfma16x16x32(kb, S16[kk][it], U[tt][it]);
          }
        }
      }
      // erase: R~ = 2^-E V - e^G (K S_reg^T) (b is applied by the solve);
      // erase-free: U = 2^-E diag(b) V.  The 2^-E factor is exact; the
      // unscaled variant is the common one (E = 0).
      auto rhs_v = [&](auto scaled) {
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
          f32x4 be4 = *reinterpret_cast<const f32x4*>(&sm.beta[hp][16 * tt + 4 * lg]);
          const f32x4 ga4 = *reinterpret_cast<const f32x4*>(&sm.gam[hp][16 * tt + 4 * lg]);
          if constexpr (decltype(scaled)::value && !ERASE) be4 *= s_dn;
#pragma unroll
          for (int it = 0; it < NIT; ++it) {
            const u16x4 vx = lds_tr4(xv, 2 * (16 * tt * kWS + 16 * it));
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              float vv = raw_to_f32<TI>(vx[r]);
              if constexpr (decltype(scaled)::value && ERASE) vv *= s_dn;
              U[tt][it][r] = ERASE ? fmaf(-ga4[r], U[tt][it][r], vv) : vv * be4[r];
            }
            // pinned in fp32: the solve rounds it to fp16, and a fused
            // FMA-with-conversion in some template instances only would make
            // the state-only and full replays differ in the last bit
            asm volatile("" : "+v"(U[tt][it]));
          }
        }
      };
      if (sexp == 0) rhs_v(std::false_type{});
      else rhs_v(std::true_type{});
      tr_keep(xv);
      if (ERASE) {
        // ---- block forward substitution (I + A) U = diag(b) R~, this wave's
        // columns.  Block row i: U_i = [(I + A_ii)^{-1} diag(b_i)] (R~_i +
        // sum_{m<i} (-A~_im) U_m); the solved rows return as fp16 B operands.
        f16x4 Yh[3][NIT];
#pragma unroll
        for (int bi = 0; bi < 4; ++bi) {
          pf_next(1);
          f32x4 X[NIT];
#pragma unroll
          for (int it = 0; it < NIT; ++it) X[it] = U[bi][it];
          const _Float16* arow = &sm.a[hp][(16 * bi + lr) * kAS];
          if (bi == 1) {
            const f16x4 a4 = lds4(arow + 8 * lg);
#pragma unroll
            for (int it = 0; it < NIT; ++it) X[it] = mfma16x16x16(a4, Yh[0][it], X[it]);
          } else if (bi >= 2) {
            const f16x8 a8 = lds8(arow + 8 * lg);
#pragma unroll
            for (int it = 0; it < NIT; ++it) X[it] = mfma16x16x32(a8, cat44(Yh[0][it], Yh[1][it]), X[it]);
            if (bi == 3) {
              // the third term as a K = 32 product with zero upper k-slots:
              // accumulating a 16x16x16 MFMA onto a 16x16x32 result (or the
              // reverse) reads two stale accumulator registers on gfx950 unless
              // about five wait states separate them, which the compiler does
              // not insert; same-shape accumulation chains are safe
              const f16x4 z4 = {};
              const f16x8 a8z = cat44(lds4(arow + 32 + 8 * lg), z4);
#pragma unroll
              for (int it = 0; it < NIT; ++it) X[it] = mfma16x16x32(a8z, cat44(Yh[2][it], z4), X[it]);
            }
          }
          const f16x4 t4 = lds4(&sm.td[hp][bi * 256 + lr * 16 + 4 * lg]);
#pragma unroll
          for (int it = 0; it < NIT; ++it) {
            U[bi][it] = mfma16x16x16(t4, to_f16x4(X[it]), f32x4{0.f, 0.f, 0.f, 0.f});
            if (bi < 3) Yh[bi][it] = to_f16x4(U[bi][it]);
          }
        }
      }
      pf_next(kSlots);  // whatever is left
  };
  auto part2 = [&](ChunkSmem<D, HP>& sm, int c0) {
    const int nv = min(kC, t_end - c0);
      // U as fp16 B operands: plain (output) and scaled by e^{G_C-G} (state)
      f16x8 U16[2][NIT], UD[2][NIT];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int it = 0; it < NIT; ++it) {
          f32x4 lo = U[2 * ks][it], hi = U[2 * ks + 1][it];
          if (want_o) U16[ks][it] = to_f16x8(lo, hi);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            lo[r] *= sm.dec[hp][32 * ks + 4 * lg + r];
            hi[r] *= sm.dec[hp][32 * ks + 16 + 4 * lg + r];
          }
          UD[ks][it] = to_f16x8(lo, hi);
          // materialise the fp16 copies here so the fp32 U dies now instead of
          // staying live through the output product
          asm volatile("" : "+v"(UD[ks][it]));
          if (want_o) asm volatile("" : "+v"(U16[ks][it]));
        }

      // ---- O^T = S Q^T diag(e^G) + U^T (P o Q K^T)^T, two token tiles at a
      // time.  Computing the transpose puts 4 consecutive value columns of one
      // token in each lane, so every lane stores 8 contiguous bytes.
      if (want_o) {
#pragma unroll
        for (int tp = 0; tp < 2; ++tp) {
          f32x4 O[2][NIT];  // tile (u, it): value rows w*IW+16it+4lg+r, token column
#pragma unroll
          for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int it = 0; it < NIT; ++it) O[u][it] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kk = 0; kk < NKJ; ++kk) {
#pragma unroll
            for (int u = 0; u < 2; ++u) {
              const int t = 16 * (2 * tp + u) + lr;
              const f16x8 qb = lds8(&sm.q[qidx<D>(t, 32 * kk + 8 * lg)]);
#pragma unroll
              for (int it = 0; it < NIT; ++it) O[u][it] = mfma16x16x32(S16[kk][it], qb, O[u][it]);
            }
          }
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const int tt = 2 * tp + u;
            const int t = 16 * tt + lr;
            const float gt = a.scale * sm.gam[hp][t];
#pragma unroll
            for (int it = 0; it < NIT; ++it) O[u][it] *= gt;
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
              if (32 * ks > 16 * tt + 15) continue;  // P o QK^T is lower triangular
              const _Float16* pr = &sm.pqk[hp][t * kPS + 32 * ks];
              const f16x8 pb = lds8(pr + 8 * lg);
#pragma unroll
              for (int it = 0; it < NIT; ++it) O[u][it] = mfma16x16x32(U16[ks][it], pb, O[u][it]);
            }
            if (sexp != 0) {  // back from the state's units (exact)
#pragma unroll
              for (int it = 0; it < NIT; ++it) O[u][it] *= s_up;
            }
            if (t < nv) {
              // uniform base (this chunk, this head) + 32-bit lane offset
              constexpr unsigned kOB = std::is_same<TO, F32>::value ? 4u : 2u;
              char* ob0 = static_cast<char*>(a.o) + (static_cast<size_t>(c0) * a.h_v + h) * D * kOB;
              const unsigned oo = kOB * (static_cast<unsigned>(t) * static_cast<unsigned>(a.h_v) * D +
                                         static_cast<unsigned>(col0 + wq * IW + 4 * lg));
#pragma unroll
              for (int it = 0; it < NIT; ++it) store4<TO>(ob0 + oo + kOB * 16 * it, 0, O[u][it]);
            }
          }
        }
      }

      // ---- S^T <- e^{G_C} S^T + K^T diag(e^{G_C-G}) U -----------------------
      {
        const float gC = sm.gam[hp][kC - 1];
        const uint32_t sb = tr_base(lds_addr(sm.k) + 2 * tro);
#pragma unroll
        for (int jt = 0; jt < NJT; ++jt) {
          SR_SCHED_FENCE();
#pragma unroll
          for (int it = 0; it < NIT; ++it) S[jt][it] *= gC;
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) {
            // K^T rows kkey(jt, ..), token k-slots {32ks+4lg.., 32ks+16+4lg..}
            constexpr int KS = ChunkSmem<D, HP>::kKS;
            const int kc = kkey(jt, 0, 0);
            const f16x8 av = cat44(as_f16x4(lds_tr4(sb, 2 * (32 * ks * KS + kc))),
                                   as_f16x4(lds_tr4(sb, 2 * ((32 * ks + 16) * KS + kc))));
#pragma unroll
            for (int it = 0; it < NIT; ++it) S[jt][it] = mfma16x16x32(av, UD[ks][it], S[jt][it]);
          }
        }
        tr_keep(sb);
      }
  };

  if constexpr (!PC) {
    for (int c0 = t_begin; c0 < t_end; c0 += kC) {
      coords();
      stage(smb[0]);
      __syncthreads();
      // the next chunk's gates, K, Q and V fly while this one computes
      const bool more = c0 + kC < t_end;
      pfn = 0;
      pf_more = more;
      pf_c0 = c0 + kC;
      if (more) pf_gates(c0 + kC);
      pf_next(2);
      tiles(smb[0]);
      __syncthreads();
      part1(smb[0]);
      part2(smb[0], c0);
      if (more) prepare(c0 + kC);
      __syncthreads();  // LDS reused by the next chunk
    }
  } else {
    // period p: the producers prepare, stage and tile chunk p in buffer
    // p & 1 and request chunk p + 1; the consumers run chunk p - 1 from
    // buffer (p - 1) & 1.  Each side has its own loop (so neither holds the
    // other's registers: the state, the prefetched rows), and both pass the
    // same two barriers per period.
    const int nch = (t_end - t_begin + kC - 1) / kC;
    if (w >= NW * HP) {
      for (int p = 0; nch > 0 && p <= nch; ++p) {
        const int pc0 = t_begin + p * kC;
        coords();
        if (p < nch) {
          if (p > 0) prepare(pc0);
          stage(smb[p & 1]);
          if (p + 1 < nch) prefetch_all(pc0 + kC);
        }
        __syncthreads();
        if (p < nch) tiles(smb[p & 1]);
        __syncthreads();
      }
      return;  // producers hold no state
    }
    for (int p = 0; nch > 0 && p <= nch; ++p) {
      const int pc0 = t_begin + p * kC;
      coords();
      if (p > 0) part1(smb[(p - 1) & 1]);
      __syncthreads();
      if (p > 0) part2(smb[(p - 1) & 1], pc0 - kC);
      __syncthreads();
    }
  }

  const float s_fin = ldexpf(1.0f, sexp);  // S = 2^E S_reg (exact)
#pragma unroll
  for (int jt = 0; jt < NJT; ++jt)
#pragma unroll
    for (int it = 0; it < NIT; ++it)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int j = kkey(jt, lg, r);
        const int i = col0 + wq * IW + 16 * it + lr;
        a.s_out[sbase + static_cast<size_t>(j) * D + i] = S[jt][it][r] * s_fin;
      }
}

template <int D, typename TI, typename TO, int HP, int NW, int VS, bool PC = false>
hipError_t launch4(const GdnArgs& a, hipStream_t s) {
  const int units = a.n_seqs * (a.h_v / HP) * VS;
  int per_xcd = (units + kXcd - 1) / kXcd;
  // longest-first order: XCD x takes the sequences of ranks x, x + 8, ...
  if (lpt_launch<PC>(a.n_seqs)) {
    const int lpt_per_xcd = (a.h_v / HP) * ((a.n_seqs + kXcd - 1) / kXcd);
    if (lpt_per_xcd > per_xcd) per_xcd = lpt_per_xcd;
  }
  dim3 grid(per_xcd * kXcd), block(64 * (NW * HP + (PC ? kProducers : 0)));
  const bool o = a.o != nullptr;
  if (a.erase && o)
    hipLaunchKernelGGL((gdn_chunk_kernel<D, TI, TO, true, true, HP, NW, VS, PC>), grid, block, 0, s, a, per_xcd);
  else if (a.erase)
    hipLaunchKernelGGL((gdn_chunk_kernel<D, TI, TO, true, false, HP, NW, VS, PC>), grid, block, 0, s, a, per_xcd);
  else if (o)
    hipLaunchKernelGGL((gdn_chunk_kernel<D, TI, TO, false, true, HP, NW, VS, PC>), grid, block, 0, s, a, per_xcd);
  else
    hipLaunchKernelGGL((gdn_chunk_kernel<D, TI, TO, false, false, HP, NW, VS, PC>), grid, block, 0, s, a, per_xcd);
  return hipGetLastError();
}

// Launch shape by the number of (sequence, value head) chains:
//  * two value heads per workgroup where the value heads of a key head pair
//    up and there are at least two chains per compute unit;
//  * at most half a chain per CU (d = 128): each chain's value columns split
//    over two workgroups (the key-side tiles are formed by both), so the
//    launch fills the CUs (4 x 32 chains: 118 instead of 128 us with
//    outputs, 87 instead of 102 us state-only).  Each workgroup is in the
//    producer/consumer form: its 4 consumer waves (16 value columns each)
//    run chunk c while 4 producer waves stage chunk c + 1 and form its tiles
//    (4 x 32 chains: 86 instead of 111 us, 57 instead of 77 us state-only;
//    the same form with one workgroup per chain, 32 columns per consumer
//    wave, measured 3.7x slower at 8 x 32 chains);
//  * up to one chain per CU (d = 128): the producer/consumer form with 8
//    consumer waves (16 value columns each, two per SIMD) and 4 producer
//    waves (8 x 32 chains without erasure: 139 against 144 us for 8 plain
//    waves; the two-workgroup split measured 168 us there);
//  * otherwise one head of 4 waves.
template <int D, typename TI, typename TO>
hipError_t launch3(const GdnArgs& a, hipStream_t s) {
  const int chains = a.n_seqs * a.h_v;
  if ((a.h_v / a.h_k) % 2 == 0 && chains >= 2 * kGfx950Cus) return launch4<D, TI, TO, 2, 4, 1>(a, s);
  if constexpr (D == 128) {  // 16 value columns per wave (d = 64 would leave 8)
    if (2 * chains <= kGfx950Cus) return launch4<D, TI, TO, 1, 4, 2, true>(a, s);
    if (chains <= kGfx950Cus) return launch4<D, TI, TO, 1, 8, 1, true>(a, s);
  }
  return launch4<D, TI, TO, 1, 4, 1>(a, s);
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
