// frag.h -- wave64 MFMA fragment algebra for gfx950 (CDNA4).
//
// Every dense product in this library is built from one primitive: a 16x16
// output tile accumulated over a 32-deep slice of the contraction,
//     D[m][n] += sum_k A[m][k] * B[k][n].
// bf16 operands use one v_mfma_f32_16x16x32_bf16; fp32 operands use eight
// v_mfma_f32_16x16x4_f32 (so the fp32 path never rounds below fp32).
//
// Operand fragments.  Lane l (li = l % 16, lg = l / 16) holds 8 values of a
// matrix X: index row (li) of a 16-row block and 8 positions of a 32-wide
// contraction block.  The position held in element e is
//     kslot(lg, e) = 4 lg + e        (e < 4)
//                  = 16 + 4 lg + e-4 (e >= 4).
// The same slot map is used for both operands of every MFMA, so the product
// is exact regardless of the hardware's own k order.  "F(X; a, b)" below
// means fragments of X whose index dimension is a and contraction dimension
// is b.  Loaded from a row-major X[a][b] (b contiguous) a fragment is two
// 4-element vector loads.
//
// Accumulators.  Lane l holds D[4 lg + q][li], q = 0..3.  Two vertically
// adjacent accumulator tiles (rows 32 kb + 0..15 and 32 kb + 16..31) hold,
// in lane l, rows 32 kb + kslot(lg, e) of column li: converted to the operand
// type they are exactly F(D; column, row), the fragment of D^T.  Products
// therefore chain in registers: the output of one MFMA product is the
// operand of the next, transposed for free.  An MFMA against an identity
// fragment turns a row-major fragment into the other orientation (exact).
//
// Fragment-native storage: a tensor consumed as fragments is stored as
// records of 64 lanes x 8 elements, lane-major, so a wave loads a fragment
// with one fully coalesced 16-byte-per-lane access.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

template <typename E> struct VecT;
template <> struct VecT<bf16> { using x8 = bf16x8; using x4 = bf16x4; };
template <> struct VecT<float> { using x8 = f32x8; using x4 = f32x4; };
template <typename E> using frag_t = typename VecT<E>::x8;
template <typename E> using quad_t = typename VecT<E>::x4;

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }
// The wave index, as a scalar: it is one value per wave, and addresses, trip
// counts and branches derived from it then stay in scalar registers.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

__device__ __forceinline__ constexpr int kslot(int lg, int e) {
  return e < 4 ? 4 * lg + e : 16 + 4 * lg + (e - 4);
}

// ---- MFMA ---------------------------------------------------------------
__device__ __forceinline__ f32x4 mma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// fp32: two independent accumulation chains (even and odd k-steps), summed
// at the end, so consecutive MFMAs do not wait on each other's results
__device__ __forceinline__ f32x4 mma(f32x8 a, f32x8 b, f32x4 c) {
  f32x4 d = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int e = 0; e < 8; e += 2) {
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[e], b[e], c, 0, 0, 0);
    d = __builtin_amdgcn_mfma_f32_16x16x4f32(a[e + 1], b[e + 1], d, 0, 0, 0);
  }
  return c + d;
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// 16-deep products over one half of a fragment's contraction slots (a quad:
// elements 0..3 or 4..7 of each lane's fragment, as the 32-deep products above
// pair them): one v_mfma_f32_16x16x16_bf16, or four v_mfma_f32_16x16x4_f32.
// Equal to the 32-deep product of the fragments with the other half zero.
typedef short i16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ f32x4 mma16(bf16x4 a, bf16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4, a), __builtin_bit_cast(i16x4, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma16(f32x4 a, f32x4 b, f32x4 c) {
  f32x4 d = f32x4{0.f, 0.f, 0.f, 0.f};
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[0], b[0], c, 0, 0, 0);
  d = __builtin_amdgcn_mfma_f32_16x16x4f32(a[1], b[1], d, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[2], b[2], c, 0, 0, 0);
  d = __builtin_amdgcn_mfma_f32_16x16x4f32(a[3], b[3], d, 0, 0, 0);
  return c + d;
}

// ---- conversions --------------------------------------------------------
template <typename E> __device__ __forceinline__ frag_t<E> to_frag(f32x4 lo, f32x4 hi);
template <> __device__ __forceinline__ bf16x8 to_frag<bf16>(f32x4 lo, f32x4 hi) {
  f32x8 t = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_convertvector(t, bf16x8);
}
template <> __device__ __forceinline__ f32x8 to_frag<float>(f32x4 lo, f32x4 hi) {
  return f32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

template <typename E> __device__ __forceinline__ quad_t<E> to_quad(f32x4 x);
template <> __device__ __forceinline__ bf16x4 to_quad<bf16>(f32x4 x) {
  return __builtin_convertvector(x, bf16x4);
}
template <> __device__ __forceinline__ f32x4 to_quad<float>(f32x4 x) { return x; }

template <typename E> __device__ __forceinline__ f32x4 quad_to_f32(quad_t<E> x);
template <> __device__ __forceinline__ f32x4 quad_to_f32<bf16>(bf16x4 x) {
  return __builtin_convertvector(x, f32x4);
}
template <> __device__ __forceinline__ f32x4 quad_to_f32<float>(f32x4 x) { return x; }

template <typename E> __device__ __forceinline__ f32x8 frag_to_f32(frag_t<E> x);
template <> __device__ __forceinline__ f32x8 frag_to_f32<bf16>(bf16x8 x) {
  return __builtin_convertvector(x, f32x8);
}
template <> __device__ __forceinline__ f32x8 frag_to_f32<float>(f32x8 x) { return x; }

template <typename E> __device__ __forceinline__ frag_t<E> f32_to_frag(f32x8 x);
template <> __device__ __forceinline__ bf16x8 f32_to_frag<bf16>(f32x8 x) {
  return __builtin_convertvector(x, bf16x8);
}
template <> __device__ __forceinline__ f32x8 f32_to_frag<float>(f32x8 x) { return x; }

template <typename E> __device__ __forceinline__ frag_t<E> zero_frag() {
  return f32_to_frag<E>(f32x8{0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f});
}

template <typename E> __device__ __forceinline__ frag_t<E> join(quad_t<E> a, quad_t<E> b) {
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

// ---- fragment loads / stores --------------------------------------------
// Natural fragment from row-major memory: `row` points at X[a0 + li][b0].
template <typename E> __device__ __forceinline__ frag_t<E> load_frag_row(const E* row, int lg) {
  quad_t<E> a = *reinterpret_cast<const quad_t<E>*>(row + 4 * lg);
  quad_t<E> b = *reinterpret_cast<const quad_t<E>*>(row + 16 + 4 * lg);
  return join<E>(a, b);
}

// Fragment-native record: 64 lanes x 8 elements.
template <typename E> __device__ __forceinline__ frag_t<E> load_rec(const E* rec, int lane) {
  return *reinterpret_cast<const frag_t<E>*>(rec + 8 * lane);
}
template <typename E> __device__ __forceinline__ void store_rec(E* rec, int lane, frag_t<E> f) {
  *reinterpret_cast<frag_t<E>*>(rec + 8 * lane) = f;
}
// The same store with the non-temporal hint, for records that nothing reads
// for a while: they go to HBM rather than staying dirty in the caches, where
// they would be evicted (written back) in the middle of later kernels' reads.
template <typename E> __device__ __forceinline__ void store_rec_nt(E* rec, int lane, frag_t<E> f) {
  constexpr int NP = (int)sizeof(frag_t<E>) / 16;   // 16-byte pieces: 1 (bf16) or 2 (fp32)
  static_assert(NP * 16 == (int)sizeof(frag_t<E>), "a fragment is whole 16-byte pieces");
  const i32x4* src = reinterpret_cast<const i32x4*>(&f);
  i32x4* dst = reinterpret_cast<i32x4*>(rec + 8 * lane);
#pragma unroll
  for (int i = 0; i < NP; ++i) __builtin_nontemporal_store(src[i], dst + i);
}
// Four converted values to dst with the non-temporal hint (one 8-byte
// store for bf16, one 16-byte store for fp32), for outputs whose next reader
// is another kernel.
template <typename E> __device__ __forceinline__ void store_quad_nt(E* dst, f32x4 x) {
  const quad_t<E> v = to_quad<E>(x);
  if constexpr (sizeof(quad_t<E>) == 8) {
    __builtin_nontemporal_store(*reinterpret_cast<const long long*>(&v), reinterpret_cast<long long*>(dst));
  } else {
    __builtin_nontemporal_store(*reinterpret_cast<const i32x4*>(&v), reinterpret_cast<i32x4*>(dst));
  }
}
// Accumulator-native record: 64 lanes x 4 elements.
template <typename E> __device__ __forceinline__ f32x4 load_acc(const E* rec, int lane) {
  return quad_to_f32<E>(*reinterpret_cast<const quad_t<E>*>(rec + 4 * lane));
}
template <typename E> __device__ __forceinline__ void store_acc(E* rec, int lane, f32x4 x) {
  *reinterpret_cast<quad_t<E>*>(rec + 4 * lane) = to_quad<E>(x);
}

// Identity fragment F(I; a, b) for an index block a whose 16 rows fall in
// half `hsel` (0: slots 0..15, 1: slots 16..31) of its contraction block.
template <typename E> __device__ __forceinline__ frag_t<E> ident_frag(int hsel, int li, int lg) {
  f32x8 t = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (lg == (li >> 2)) t[4 * hsel + (li & 3)] = 1.f;
  return f32_to_frag<E>(t);
}

// The 16 x 16 identity as a quad operand of mma16 (either half)
template <typename E> __device__ __forceinline__ quad_t<E> ident_quad(int li, int lg) {
  f32x4 t = {0.f, 0.f, 0.f, 0.f};
  if (lg == (li >> 2)) t[li & 3] = 1.f;
  return to_quad<E>(t);
}

__device__ __forceinline__ f32x4 scale4(f32x4 x, float s) {
  return f32x4{x[0] * s, x[1] * s, x[2] * s, x[3] * s};
}

// Wave-wide inclusive prefix sum over the 64 lanes.
__device__ __forceinline__ float wave_incl_scan(float x, int lane) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    float t = __shfl_up(x, off, 64);
    if (lane >= off) x += t;
  }
  return x;
}

// Cross-lane reductions on the VALU (no LDS crossbar traffic).  Every lane
// ends with the same bits: each step adds a value to its mirror image, and
// both partners add the same two operands.
template <int CTRL> __device__ __forceinline__ float dpp_mov(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
// Sum over the four lane groups (lanes li, li+16, li+32, li+48): the
// permlane16 swap pairs rows 2k and 2k+1, the permlane32 swap the halves.
__device__ __forceinline__ float sum_groups(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}
// Sum over the 16 lanes of a group: DPP quad permutes (lane ^ 1, lane ^ 2),
// then the half-row mirror (quad q <-> q ^ 1) and the row mirror (halves).
__device__ __forceinline__ float sum_in_group(float x) {
  x += dpp_mov<0xB1>(x);
  x += dpp_mov<0x4E>(x);
  x += dpp_mov<0x141>(x);
  x += dpp_mov<0x140>(x);
  return x;
}

}  // namespace gdn

namespace gdn {

// ---- natural tiles staged in LDS ----------------------------------------
// A 64 x D tile of a token-major tensor (rows = tokens of one chunk, one
// head) in LDS: row r at r * RB bytes (RB = D * sizeof(E)), its 16-byte
// chunks XOR-swizzled by the row (chunk c stored at c ^ (r % NCH)) so that
// the 16 rows of a fragment read hit distinct banks.
template <typename E, int D>
struct NatTile {
  static constexpr int RB = D * (int)sizeof(E);
  static constexpr int NCH = RB / 16;
  static constexpr int BYTES = 64 * RB;
  __device__ static __forceinline__ int off(int r, int byte) {
    return r * RB + ((((byte >> 4) ^ (r & (NCH - 1))) << 4) | (byte & 15));
  }
};

// A 16-byte piece of a row (8 bf16 or 4 fp32 values) times s, rounded back
// to the element type: the row normalisation every kernel applies alike.
template <typename E> __device__ __forceinline__ i32x4 scale_piece(i32x4 v, float s);
template <> __device__ __forceinline__ i32x4 scale_piece<bf16>(i32x4 v, float s) {
  f32x8 f = __builtin_convertvector(__builtin_bit_cast(bf16x8, v), f32x8);
#pragma unroll
  for (int e = 0; e < 8; ++e) f[e] *= s;
  return __builtin_bit_cast(i32x4, __builtin_convertvector(f, bf16x8));
}
template <> __device__ __forceinline__ i32x4 scale_piece<float>(i32x4 v, float s) {
  f32x4 f = __builtin_bit_cast(f32x4, v);
#pragma unroll
  for (int e = 0; e < 4; ++e) f[e] *= s;
  return __builtin_bit_cast(i32x4, f);
}
// Sum of squares of the values of a 16-byte piece, in element order.
template <typename E> __device__ __forceinline__ float sum_sq_piece(i32x4 v);
template <> __device__ __forceinline__ float sum_sq_piece<bf16>(i32x4 v) {
  const f32x8 f = __builtin_convertvector(__builtin_bit_cast(bf16x8, v), f32x8);
  float s = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) s += f[e] * f[e];
  return s;
}
template <> __device__ __forceinline__ float sum_sq_piece<float>(i32x4 v) {
  const f32x4 f = __builtin_bit_cast(f32x4, v);
  float s = 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) s += f[e] * f[e];
  return s;
}
// The same for a fragment (8 values of one row).
template <typename E> __device__ __forceinline__ frag_t<E> scale_frag(frag_t<E> x, float s) {
  f32x8 f = frag_to_f32<E>(x);
#pragma unroll
  for (int e = 0; e < 8; ++e) f[e] *= s;
  return f32_to_frag<E>(f);
}
// Reciprocal row norms carry the branch of the normalisation in their sign:
// positive 1 / ||x|| where ||x|| exceeds the floor, -1 / floor below it;
// the row scale is the absolute value.

// One thread's share of a staged tile, NTHR threads per tile: load() issues
// every global read of rows [0, L) of X (row r at src + r * rstride
// elements; rows >= L, and with `width` < D the columns past it, read as
// zero: a narrower tensor padded with zeros to D), store() writes the
// swizzled LDS tile.
// With `rs`, row r is scaled by |rs[r * rsstride]| on its way to LDS (the
// scale reads are issued with the tile's, rows >= L read row 0's and scale
// zeros).  Loading several tiles before storing any keeps all their reads
// in flight; L >= 1.
template <typename E, int D, int NTHR>
struct TileStage {
  using T = NatTile<E, D>;
  static constexpr int N = 64 * T::NCH;   // 16-byte pieces of the tile
  static_assert(N % NTHR == 0, "tile pieces must divide over the threads");
  static constexpr int PER = N / NTHR;
  i32x4 v[PER];
  float sc[PER];
  bool scaled = false;
  __device__ __forceinline__ void load(const E* src, size_t rstride, int L, int tid,
                                       const float* rs = nullptr, size_t rsstride = 0, int width = D) {
    const int wp = width * (int)sizeof(E) / 16;   // 16-byte pieces of a row that exist
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int q = tid + k * NTHR, r = q / T::NCH, c = q - r * T::NCH;
      v[k] = i32x4{0, 0, 0, 0};
      if (r < L && c < wp) v[k] = *reinterpret_cast<const i32x4*>(reinterpret_cast<const char*>(src + (size_t)r * rstride) + 16 * c);
    }
    scaled = rs != nullptr;
    if (rs) {
#pragma unroll
      for (int k = 0; k < PER; ++k) {
        const int q = tid + k * NTHR, r = q / T::NCH;
        sc[k] = rs[(size_t)(r < L ? r : 0) * rsstride];   // sign-encoded, as stored
      }
    }
  }
  // With row scales: the first lane of each row writes its (sign-encoded)
  // scale to dst[r], rows >= L included.  No barrier.
  __device__ __forceinline__ void store_scales(float* dst, int tid) const {
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int q = tid + k * NTHR, r = q / T::NCH, c = q - r * T::NCH;
      if (c == 0) dst[r] = sc[k];
    }
  }
  // L2-normalise the loaded rows (waits for the reads): each row's pieces
  // sit in NCH consecutive lanes, whose sums of squares are combined by a
  // butterfly; the rows are scaled on their way to LDS.  With `inv`, the
  // first lane of each row r < L writes its sign-encoded reciprocal norm to
  // inv[r * stride].
  __device__ __forceinline__ void norm_rows(int L, int tid, float* inv, size_t stride) {
    static_assert(64 % T::NCH == 0 && NTHR % 64 == 0, "a row's pieces must sit in one wave");
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int q = tid + k * NTHR, r = q / T::NCH, c = q - r * T::NCH;
      float ss = sum_sq_piece<E>(v[k]);
#pragma unroll
      for (int off = T::NCH / 2; off > 0; off >>= 1) ss += __shfl_xor(ss, off, 64);
      const float n = sqrtf(ss);
      const float iv = n > 1e-12f ? 1.f / n : -1.f / 1e-12f;
      sc[k] = iv;
      if (inv && c == 0 && r < L) inv[(size_t)r * stride] = iv;
    }
    scaled = true;
  }
  __device__ __forceinline__ void store(char* tile, int tid) const {
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int q = tid + k * NTHR, r = q / T::NCH, c = q - r * T::NCH;
      *reinterpret_cast<i32x4*>(tile + T::off(r, 16 * c)) = scaled ? scale_piece<E>(v[k], fabsf(sc[k])) : v[k];
    }
  }
};

// Zero the six 16 x 16 blocks strictly above (UPPER: column block > row
// block) or strictly below the block diagonal of a 64 x 64 LDS matrix of X
// (row stride ld elements, rows 16-byte aligned), one 16-byte store per
// piece, spread over nthr threads.  No barrier.
template <typename X, bool UPPER>
__device__ __forceinline__ void zero_off_blocks(X* M, int ld, int tid, int nthr) {
  constexpr int PR = 16 * (int)sizeof(X) / 16;   // pieces per block row
  constexpr int N = 6 * 16 * PR;
  for (int e = tid; e < N; e += nthr) {
    const int b = e / (16 * PR), rem = e - b * 16 * PR, rr = rem / PR, pc = rem - rr * PR;
    const int hi = b < 1 ? 1 : (b < 3 ? 2 : 3), lo = b - hi * (hi - 1) / 2;
    const int br = UPPER ? lo : hi, bc = UPPER ? hi : lo;
    *reinterpret_cast<i32x4*>(reinterpret_cast<char*>(M + (16 * br + rr) * ld + 16 * bc) + 16 * pc) = i32x4{0, 0, 0, 0};
  }
}

// Natural fragment F(X; s, i) (index row 16*ab + li, contraction 32*kb..) from a staged tile.
template <typename E, int D>
__device__ __forceinline__ frag_t<E> tile_frag(const char* tile, int ab, int kb, int li, int lg) {
  using T = NatTile<E, D>;
  const int r = 16 * ab + li;
  const int b0 = (32 * kb + 4 * lg) * (int)sizeof(E);
  const int b1 = (32 * kb + 16 + 4 * lg) * (int)sizeof(E);
  const quad_t<E> a = *reinterpret_cast<const quad_t<E>*>(tile + T::off(r, b0));
  const quad_t<E> b = *reinterpret_cast<const quad_t<E>*>(tile + T::off(r, b1));
  return join<E>(a, b);
}

}  // namespace gdn
