// bwd.hip -- backward kernels of the gated delta rule (chunked form).
//
// Per chunk, with the forward quantities of fwd.hip (gamma, D, A, T, W, U,
// V', entering state h) and H' = dL/dh' (gradient of the state leaving the
// chunk), and Q scaled by `scale`:
//   dV'  = P^T dO + Kt H'                  P = (Q K^T) * D, lower incl. diagonal
//   dh   = exp(gamma_L) H' + (Gam Q)^T dO - W^T dV'     (becomes H' of the previous chunk)
//          (Z = (Gam Q)^T dO depends only on the chunk and is precomputed in K4)
//   dP   = dO V'^T (lower)
//   dQ   = Gam dO h^T + (dP * D) K
//   dK   = (dP * D)^T Q + diag(exp(gamma_L - gamma)) V' H'^T + diag(beta Gam) T^T dW
//          + (E + E^T) K,      E = dA * beta_r D (strict lower)
//   dW   = -dV' h^T,  dU = dV',  dT = dW Xw^T + dU Xu^T  (Xw = diag(beta Gam) K, Xu = diag(beta) V)
//   dA   = strict_lower(-T^T dT T^T)
//   dV   = diag(beta) T^T dU
//   dbeta_r = Gam_r k_r.(T^T dW)_r + v_r.(T^T dU)_r + sum_s dA_rs (K K^T * D)_rs
// Two of these are formed without dW and dT: since V' = T (Xu - Xw h),
// dT = dV' (Xu - Xw h)^T = (dV' V'^T)(I + A)^T, and T (I + A) = I, so
//   dA   = strict_lower(-T^T (dV' V'^T)),   T^T dW = -(T^T dV') h^T.
// dbeta has a second form: with B = diag(beta) invertible, V' = (B^-1 +
// A')^-1 (V - Gam K h) (A = B A'), so differentiating B^-1 gives
//   dbeta_r = (T^T dV')_r . V'_r / beta_r.
// The two agree exactly but round differently: V' is held in the operand
// type, and its rounding reaches the sum through sum_s dA_rs A_rs (dA_rs =
// -(T^T dV')_r . V'_s), the quotient through V'_r alone.  Row by row the
// kernel takes the quotient where ||A_r||^2 = sum_s A_rs^2 exceeds 1 (keys
// that cluster, where the sum's terms cancel) and the sum elsewhere (which
// includes beta_r = 0, where A_r vanishes).
//   dgamma collects the decay terms (output, P, Xw, A, Kt and the state decay);
//   dg_s = sum_{r >= s} dgamma_r within the chunk.
// These are the reverse-mode equations of the chunked forward; the kernel
// split follows the native family in the XTuner / Ascend 910C article
// (section 3.1.2, Fig. 7): a local dv step (K4), the reverse pass through the
// state-transition chain (K5) and the dq/dk/dw/dg projection with the WY
// backward folded in (K6).
#include "frag.h"
#include "gdn_internal.h"
#include "ring.h"

namespace gdn {

// Per-wave work lists packed into an integer: item k of wave w is nibble
// (w * MAXT + k) (15 = none), built from an owner table at compile time, so
// a wave walks only its own items and the code holds MAXT copies of a body
// rather than one per item.
template <int NI, int NWV, int MAXT>
constexpr unsigned long long pack_owned(const int (&own)[NI]) {
  unsigned long long r = ~0ull;
  for (int w = 0; w < NWV; ++w) {
    int k = 0;
    for (int t = 0; t < NI; ++t)
      if (own[t] == w && k < MAXT) {
        const int sh = 4 * (w * MAXT + k);
        r = (r & ~(15ull << sh)) | ((unsigned long long)t << sh);
        ++k;
      }
  }
  return r;
}
__device__ __forceinline__ int owned_item(unsigned long long packed, int w, int maxt, int k) {
  return (int)((packed >> (4 * (w * maxt + k))) & 15ull);
}
// Row and column block of the t-th lower 16 x 16 tile of a 64 x 64 matrix
// (row-major order over the lower triangle including the diagonal).
__device__ __forceinline__ int tri_row(int t) { return t >= 6 ? 3 : (t >= 3 ? 2 : (t >= 1 ? 1 : 0)); }
__device__ __forceinline__ int tri_col(int t) { const int r = tri_row(t); return t - r * (r + 1) / 2; }

// --------------------------------------------------------------------------
// K4: per (chunk, head), D/32 waves; wave w owns feature columns [32w, 32w+32).
// Writes the operands of the reverse pass:
//   Ktn = F(Kt; s, i), WnT = F(-W; i, r)            (fragment-native)
//   Z   = (scale Gam Q)^T dO   [jb][ib] accumulator records, operand type
//   dVl = P^T dO               [jb][sb] accumulator records, operand type
template <typename E, int D>
struct BwdPrepSmem {
  static constexpr int NJ = D / 16;
  static constexpr int TILE = NatTile<E, D>::BYTES;
  static constexpr int LDE = sizeof(E) == 2 ? 72 : 68;
  static constexpr int oQ = 0;
  static constexpr int oK = oQ + TILE;
  static constexpr int oO = oK + TILE;
  static constexpr int oDof = oO + TILE;                         // F(dO; j, r) records [jb][rkb]
  static constexpr int oPT = oDof + NJ * 2 * REC * (int)sizeof(E);  // P^T [s][r], operand type
  static constexpr int oG = oPT + 64 * LDE * (int)sizeof(E);
  static constexpr int BYTES = oG + 256;
};

template <typename E, int D, bool NORM>
__global__ __launch_bounds__(64 * (D / 32)) void k_bwd_prep(Params p) {
  using S = BwdPrepSmem<E, D>;
  constexpr int KB = D / 32, NJ = D / 16, NW = D / 32, LDE = S::LDE;
  __shared__ __attribute__((aligned(16))) char smem[S::BYTES];
  char* tQ = smem + S::oQ;
  char* tK = smem + S::oK;
  char* tO = smem + S::oO;
  E* s_dof = reinterpret_cast<E*>(smem + S::oDof);
  E* sPT = reinterpret_cast<E*>(smem + S::oPT);
  float* s_gam = reinterpret_cast<float*>(smem + S::oG);
  // units in reverse chunk order: the reverse pass reads the last chunk
  // first, and it is then the least recently written (the caches keep the
  // order of use)
  const int ch = p.NC * p.H - 1 - (int)blockIdx.x;
  const int H = p.H;
  const int c = ch / H, h = ch - c * H;
  const int4 ct = chunk_info(p, c);
  const int tok0 = ct.x, L = ct.y;
  const int lane = lane_id(), w = wave_id(), li = lane & 15, lg = lane >> 4;
  const int tid = threadIdx.x;
  constexpr int NT = 64 * NW;
  const E* Wn = reinterpret_cast<const E*>(p.Wn);
  E* Ktn = reinterpret_cast<E*>(p.Ktn);
  E* WnT = reinterpret_cast<E*>(p.WnT);
  // dO: [tokens][H][dv], contiguous
  const size_t rowstride = (size_t)H * p.vdim;
  const size_t base = ((size_t)tok0 * H + h) * p.vdim;
  const float sc = p.scale;

  // ---- stage Q, K, dO; the -W records of this wave's i-slice.  Every global
  // read is issued before the first use of any of them.
  const float gv = p.gamma[(size_t)ch * 64 + lane];
  frag_t<E> wrec[4];
  {
    TileStage<E, D, NT> sq, sk, so;
    const size_t nb = (size_t)tok0 * H + h;   // reciprocal norms of this chunk's rows, stride H
    // q, k: token stride ldq, dk wide; dO: contiguous, dv wide (zeros past the widths)
    const size_t xbase = (size_t)tok0 * p.ldq + (size_t)h * p.kdim;
    sq.load(reinterpret_cast<const E*>(p.q) + xbase, (size_t)p.ldq, L, tid, nullptr, 0, p.kdim);
    sk.load(reinterpret_cast<const E*>(p.k) + xbase, (size_t)p.ldq, L, tid, NORM ? p.kinv + nb : nullptr, H, p.kdim);
    so.load(reinterpret_cast<const E*>(p.dO) + base, rowstride, L, tid, nullptr, 0, p.vdim);
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) wrec[rb] = load_rec<E>(Wn + (((size_t)ch * 4 + rb) * KB + w) * REC, lane);
    if (w == 0) s_gam[lane] = gv;
    // query norms for this pass and the gradient pass (same arithmetic as the forward's)
    if constexpr (NORM) sq.norm_rows(L, tid, p.qinv + nb, H);
    sq.store(tQ, tid);
    sk.store(tK, tid);
    so.store(tO, tid);
  }
  __syncthreads();
  const float gL = s_gam[63];
  const frag_t<E> id0 = ident_frag<E>(0, li, lg), id1 = ident_frag<E>(1, li, lg);
  auto qf = [&](int ab, int kb) { return tile_frag<E, D>(tQ, ab, kb, li, lg); };
  auto kf = [&](int ab, int kb) { return tile_frag<E, D>(tK, ab, kb, li, lg); };
  auto of = [&](int ab, int kb) { return tile_frag<E, D>(tO, ab, kb, li, lg); };

  // Ktn records (sb, kb = w): natural key rows scaled by exp(gamma_L - gamma_s)
#pragma unroll
  for (int sb = 0; sb < 4; ++sb) {
    const int s_ = 16 * sb + li;
    f32x8 x = frag_to_f32<E>(kf(sb, w));
    const float f = __expf(gL - s_gam[s_]);
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] *= f;
    store_rec<E>(Ktn + (((size_t)ch * 4 + sb) * KB + w) * REC, lane, f32_to_frag<E>(x));
  }

  // transposes of this wave's slice of Q (scaled by scale * Gam), dO and -W
  frag_t<E> dof[2][2], qg[2][2];  // F(dO; j, r), F(scale Gam Q; i, r) for block 2w + hs, rkb
#pragma unroll
  for (int hs = 0; hs < 2; ++hs) {
    const frag_t<E> idh = hs ? id1 : id0;
    f32x4 tq[4], td[4], tw[4];
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      tq[rb] = mma(qf(rb, w), idh, zero4());
      td[rb] = mma(of(rb, w), idh, zero4());
      tw[rb] = mma(wrec[rb], idh, zero4());
      // tq lane holds Q[r = 16rb + 4lg + q][i = 32w + 16hs + li]
#pragma unroll
      for (int q = 0; q < 4; ++q) tq[rb][q] *= sc * __expf(s_gam[16 * rb + 4 * lg + q]);
    }
    const int ib = 2 * w + hs;
#pragma unroll
    for (int rkb = 0; rkb < 2; ++rkb) {
      qg[hs][rkb] = to_frag<E>(tq[2 * rkb], tq[2 * rkb + 1]);
      dof[hs][rkb] = to_frag<E>(td[2 * rkb], td[2 * rkb + 1]);
      store_rec<E>(s_dof + (ib * 2 + rkb) * REC, lane, dof[hs][rkb]);
      store_rec<E>(WnT + (((size_t)ch * NJ + ib) * 2 + rkb) * REC, lane, to_frag<E>(tw[2 * rkb], tw[2 * rkb + 1]));
    }
  }

  // P = scale (Q K^T) * D, lower incl. diagonal, one tile per wave in turn -> sPT[s][r]
  {
    constexpr int TR[10] = {0, 1, 1, 2, 2, 2, 3, 3, 3, 3};
    constexpr int TS[10] = {0, 0, 1, 0, 1, 2, 0, 1, 2, 3};
    // blocks of P^T with s-block > r-block are zero
    zero_off_blocks<E, false>(sPT, LDE, tid, NT);
#pragma unroll
    for (int t = 0; t < 10; ++t) {
      if (t % NW != w) continue;
      const int rb = TR[t], sb = TS[t];
      f32x4 acc = zero4();
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) acc = mma(qf(rb, kb), kf(sb, kb), acc);
      const int s_ = 16 * sb + li;
      const float gs = s_gam[s_];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int r = 16 * rb + 4 * lg + q;
        acc[q] = s_ <= r ? sc * acc[q] * __expf(s_gam[r] - gs) : 0.f;
      }
      // lane holds P[r = 16rb + 4lg + q][s]: four consecutive r of row s of P^T
      *reinterpret_cast<quad_t<E>*>(sPT + s_ * LDE + 16 * rb + 4 * lg) = to_quad<E>(acc);
    }
  }
  __syncthreads();

  // Z[i][j] = sum_r (scale Gam_r Q[r][i]) dO[r][j] for this wave's i-blocks, all j-blocks
#pragma unroll
  for (int jb = 0; jb < NJ; ++jb) {
    const frag_t<E> d0 = load_rec<E>(s_dof + (jb * 2 + 0) * REC, lane);
    const frag_t<E> d1 = load_rec<E>(s_dof + (jb * 2 + 1) * REC, lane);
#pragma unroll
    for (int hs = 0; hs < 2; ++hs) {
      f32x4 acc = mma(qg[hs][0], d0, zero4());
      acc = mma(qg[hs][1], d1, acc);
      store_acc<E>(reinterpret_cast<E*>(p.Z) + (((size_t)ch * NJ + jb) * NJ + 2 * w + hs) * AREC, lane, acc);
    }
  }
  // dVl[s][j] = sum_r P[r][s] dO[r][j] for this wave's j-blocks
#pragma unroll
  for (int sb = 0; sb < 4; ++sb) {
    f32x4 acc[2] = {zero4(), zero4()};
#pragma unroll
    for (int rkb = 0; rkb < 2; ++rkb) {
      if (2 * rkb + 1 < sb) continue;   // P[r][s] = 0 for r < s
      const frag_t<E> pf = load_frag_row<E>(sPT + (16 * sb + li) * LDE + 32 * rkb, lg);
#pragma unroll
      for (int hs = 0; hs < 2; ++hs) acc[hs] = mma(pf, dof[hs][rkb], acc[hs]);
    }
#pragma unroll
    for (int hs = 0; hs < 2; ++hs)
      store_acc<E>(reinterpret_cast<E*>(p.dVl) + (((size_t)ch * NJ + 2 * w + hs) * 4 + sb) * AREC, lane, acc[hs]);
  }
}

// --------------------------------------------------------------------------
// K5: reverse state-gradient pass.  One compute wave per (sequence, head,
// 16-column block jb of d_v); the d_k x 16 slice of H' stays in accumulator
// registers.  The chunk operands (Kt, -W^T, this block of Z and dVl, gamma)
// are streamed through an LDS ring by loader waves (ring.h), last chunk first;
// a workgroup holds CPW column blocks, as in the forward pass.
// Per chunk: store H' (fragment-native), dV' = dVl + Kt H', store dV',
// H' <- exp(gamma_L) H' + Z - W^T dV'.  H' and dV' are stored non-temporal:
// right after a forward, the caches hold its freshly written context, and
// these 48 MB (at 4096 x 16 x 128) written into the caches would evict it
// during this pass, whose operand reads then wait behind the write-backs.
template <typename E, int D, int CPW = 1>
struct BwdRing {
  static constexpr int KB = D / 32, NJ = D / 16;
  static constexpr int RECB = REC * (int)sizeof(E);
  static constexpr int oK = 0;
  static constexpr int oW = oK + 4 * KB * RECB;
  static constexpr int oZ = oW + NJ * 2 * RECB;
  static constexpr int ZB = NJ * AREC * (int)sizeof(E), VB = 4 * AREC * (int)sizeof(E);   // one column block
  static constexpr int oV = oZ + CPW * ZB;
  static constexpr int oG = oV + CPW * VB;
  static constexpr int SLOT = oG + 256;
  // at most four waves (one per SIMD, so a compute wave may use 512 VGPRs):
  // with two compute waves, at most two loaders and three slots
  static constexpr int S = CPW == 1 ? ring_slots(SLOT) : (ring_slots(SLOT) < 3 ? ring_slots(SLOT) : 3);
  static constexpr int WAVES = CPW + S - 1;   // compute waves, then loaders
  static constexpr bool FITS = S * SLOT <= 160 * 1024;
  static_assert(WAVES <= 4, "one wave per SIMD");
};

template <typename E, int D, bool ROT, int CPW>
__global__ __launch_bounds__((64 * BwdRing<E, D, CPW>::WAVES)) void k_bwd_state(Params p) {
  using R = BwdRing<E, D, CPW>;
  static_assert(R::FITS, "the ring fits the LDS");
  constexpr int NJ = D / 16, KB = D / 32, S = R::S;
  __shared__ __attribute__((aligned(1024))) char ring[S * R::SLOT];
  const int lane = lane_id(), w = wave_id(), li = lane & 15, lg = lane >> 4;
  const int b = blockIdx.x, xcd = b & 7, slot = b >> 3;
  // CPW column blocks per workgroup (one compute wave each), as in the forward pass
  constexpr int NJP = NJ / CPW;
  const int unit = (slot / NJP) * 8 + xcd, jbp = slot % NJP;
  const int jb0 = CPW * jbp, jb = jb0 + (CPW > 1 && w < CPW ? w : 0);
  if (unit >= p.N * p.H) return;
  const int n = unit / p.H, h = unit - n * p.H;
  const int4 st = seq_info(p, n);
  const int c0 = st.x, nc = st.y;
  // states [N][H][dk][dv]; rows past dk and columns past dv are the padding of D
  const size_t sbase = (size_t)unit * p.kdim * p.vdim;
  const bool col_real = 16 * jb < p.vdim;
  const E* Ktn = reinterpret_cast<const E*>(p.Ktn);
  const E* WnT = reinterpret_cast<const E*>(p.WnT);
  E* HPf = reinterpret_cast<E*>(p.HPf);
  E* dVf = reinterpret_cast<E*>(p.dVf);
  const int rot = jbp;   // ROT: rotated shared reads, as in the forward pass

  // step t handles chunk nc - 1 - t
  auto issue = [&](int t) {
    const size_t ch = (size_t)(c0 + nc - 1 - t) * p.H + h;
    char* sl = ring + (t % S) * R::SLOT;
    if constexpr (ROT) {
      dma_kib_rot(Ktn + ch * 4 * KB * REC, sl + R::oK, 4 * KB * R::RECB, lane, rot * (4 * KB * R::RECB / 1024) / NJP);
      dma_kib_rot(WnT + ch * NJ * 2 * REC, sl + R::oW, NJ * 2 * R::RECB, lane, rot * (NJ * 2 * R::RECB / 1024) / NJP);
    } else {
      dma_kib(Ktn + ch * 4 * KB * REC, sl + R::oK, 4 * KB * R::RECB, lane);
      dma_kib(WnT + ch * NJ * 2 * REC, sl + R::oW, NJ * 2 * R::RECB, lane);
    }
    dma_kib(reinterpret_cast<const E*>(p.Z) + (ch * NJ + jb0) * NJ * AREC, sl + R::oZ, CPW * R::ZB, lane);
    dma_kib(reinterpret_cast<const E*>(p.dVl) + (ch * NJ + jb0) * 4 * AREC, sl + R::oV, CPW * R::VB, lane);
    dma_256(p.gamma + ch * 64, sl + R::oG, lane);
  };
  if (w >= CPW && w - CPW < nc) issue(w - CPW);

  if (w < CPW) {
    f32x4 hs[NJ];
#pragma unroll
    for (int ib = 0; ib < NJ; ++ib) {
      if (p.dht && col_real && 16 * ib < p.kdim) {
        const int ld = p.vdim;
        const float* src = p.dht + sbase + (size_t)(16 * ib + 4 * lg) * ld + 16 * jb + li;
        hs[ib] = f32x4{src[0], src[ld], src[2 * ld], src[3 * ld]};
      } else {
        hs[ib] = zero4();
      }
    }
    // One chunk's LDS operands.  Where registers allow (bf16, or d = 64),
    // two sets alternate: the next chunk's set is read from its slot while
    // this chunk's second product runs.
    constexpr bool kPipe = sizeof(E) == 2 || D <= 64;
    // Values are kept as read (dVl and Z in the storage type, raw gamma_L)
    // and converted where the step uses them, so nothing in the step waits
    // for the reads of the next set.
    struct Ops {
      frag_t<E> kn[4][KB], wt[NJ][2];
      quad_t<E> dv[4], z[NJ];
      float gL;
    };
    auto read_ops = [&](Ops& o, int t) {
      const char* sl = ring + (t % S) * R::SLOT;
#pragma unroll
      for (int sb = 0; sb < 4; ++sb)
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
          o.kn[sb][kb] = load_rec<E>(reinterpret_cast<const E*>(sl + R::oK) + (sb * KB + kb) * REC, lane);
#pragma unroll
      for (int sb = 0; sb < 4; ++sb) o.dv[sb] = *reinterpret_cast<const quad_t<E>*>(reinterpret_cast<const E*>(sl + R::oV) + (CPW > 1 ? (jb - jb0) * 4 * AREC : 0) + sb * AREC + 4 * lane);
#pragma unroll
      for (int ib = 0; ib < NJ; ++ib)
#pragma unroll
        for (int rkb = 0; rkb < 2; ++rkb)
          o.wt[ib][rkb] = load_rec<E>(reinterpret_cast<const E*>(sl + R::oW) + (ib * 2 + rkb) * REC, lane);
#pragma unroll
      for (int ib = 0; ib < NJ; ++ib) o.z[ib] = *reinterpret_cast<const quad_t<E>*>(reinterpret_cast<const E*>(sl + R::oZ) + (CPW > 1 ? (jb - jb0) * NJ * AREC : 0) + ib * AREC + 4 * lane);
      o.gL = reinterpret_cast<const float*>(sl + R::oG)[63];
    };
    auto step = [&](int t, Ops& cur, Ops& nxt) {
      const size_t ch = (size_t)(c0 + nc - 1 - t) * p.H + h;
      frag_t<E> hfr[KB];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) hfr[kb] = to_frag<E>(hs[2 * kb], hs[2 * kb + 1]);
      f32x4 dv[4];
#pragma unroll
      for (int sb = 0; sb < 4; ++sb) dv[sb] = quad_to_f32<E>(cur.dv[sb]);
      // dV' = dVl + Kt H'
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int sb = 0; sb < 4; ++sb) dv[sb] = mma(cur.kn[sb][kb], hfr[kb], dv[sb]);
      // exp(gamma_L) H' + Z and dV' in the operand type, before the barrier:
      // the empty asm keeps the compiler from sinking them past it onto the
      // second product's critical path
      const float GL = __expf(cur.gL);
#pragma unroll
      for (int ib = 0; ib < NJ; ++ib) {
        hs[ib] = scale4(hs[ib], GL) + quad_to_f32<E>(cur.z[ib]);
        asm volatile("" : "+v"(hs[ib]));
      }
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) store_rec_nt<E>(HPf + ((ch * NJ + jb) * KB + kb) * REC, lane, hfr[kb]);
      frag_t<E> dvf[2];
#pragma unroll
      for (int rkb = 0; rkb < 2; ++rkb) {
        dvf[rkb] = to_frag<E>(dv[2 * rkb], dv[2 * rkb + 1]);
        asm volatile("" : "+v"(dvf[rkb]));
      }
      if (kPipe && t + 1 < nc) {
        // this chunk's reads are complete: release its slot
        wait_lds();
        ring_barrier();
      }
      // fetch the next chunk's operands (the last step reads its own slot
      // again, unused), interleaved with the second product below
      if (kPipe) read_ops(nxt, t + 1 < nc ? t + 1 : t);
      // H' <- exp(gamma_L) H' + Z - W^T dV'
#pragma unroll
      for (int rkb = 0; rkb < 2; ++rkb)
#pragma unroll
        for (int ib = 0; ib < NJ; ++ib) hs[ib] = mma(cur.wt[ib][rkb], dvf[rkb], hs[ib]);
      if (kPipe) {
#pragma unroll
        for (int i = 0; i < 2 * NJ; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);   // LDS reads
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
        }
      }
#pragma unroll
      for (int rkb = 0; rkb < 2; ++rkb) store_rec_nt<E>(dVf + ((ch * NJ + jb) * 2 + rkb) * REC, lane, dvf[rkb]);
    };
    if constexpr (kPipe) {
      if (nc > 0) {
        Ops A, B;
        ring_barrier();
        read_ops(A, 0);
        for (int t = 0; t < nc; t += 2) {
          step(t, A, B);
          if (t + 1 < nc) step(t + 1, B, A);
        }
      }
    } else {
      Ops A;
      for (int t = 0; t < nc; ++t) {
        ring_barrier();
        read_ops(A, t);
        step(t, A, A);
        wait_lds();
      }
    }
    if (p.dh0 && col_real) {
#pragma unroll
      for (int ib = 0; ib < NJ; ++ib) {
        if (16 * ib >= p.kdim) continue;
        const int ld = p.vdim;
        float* dst = p.dh0 + sbase + (size_t)(16 * ib + 4 * lg) * ld + 16 * jb + li;
        dst[0] = hs[ib][0];
        dst[ld] = hs[ib][1];
        dst[2 * ld] = hs[ib][2];
        dst[3 * ld] = hs[ib][3];
      }
    }
  } else {
    // loader wave w: steps t with t % (S - 1) == w - CPW, S - 1 ahead
    for (int t = 0; t < nc; ++t) {
      const bool mine = (t % (S - 1)) == w - CPW;
      if (mine) wait_vmem();
      ring_barrier();
      if (mine && t + S - 1 < nc) issue(t + S - 1);
    }
  }
}

// --------------------------------------------------------------------------
// K6: per (chunk, head) gradients dq, dk, dv, dbeta, dg.  D/16 waves; wave
// w owns the 16 feature columns [16w, 16w+16) of dq/dk (i) and dv (j);
// column block w is half hw = w % 2 of the 32-wide contraction block
// kw = w / 2.  Quantities that need every column (dP, G = dV' V'^T, T, dA,
// E, T^T dV') are shared through LDS, their 16 x 16 tiles dealt over the
// waves; sums over waves use per-wave slots so the result is deterministic.
template <typename E, int D>
struct BwdGradSmem {
  static constexpr int KB = D / 32;
  static constexpr int NW = D / 16;
  static constexpr int LDF = 68;                        // fp32 64x64 matrices, padded rows
  static constexpr int MAT = 64 * LDF * 4;
  static constexpr int LDE = sizeof(E) == 2 ? 72 : 68;  // operand-type 64x64 matrix
  static constexpr int PMAT = 64 * LDE * (int)sizeof(E);
  static constexpr int RECB = REC * (int)sizeof(E);
  static constexpr int SET = 4 * KB * RECB;             // records of a 64 x D fragment set
  static constexpr int TILE = NatTile<E, D>::BYTES;
  // Q and K are staged as natural tiles where they fit; in fp32 at D = 128
  // their fragments are read from global memory instead (the 64 KB of tiles
  // would take the workgroup past the 160 KB of LDS), the gradients are
  // stored straight from the waves (a staged 64 x 128 fp32 tile needs 32 KB),
  // and the transposed T and dP*D operands are read from those matrices
  // rather than from records of their own.
  static constexpr bool kStageQK = !(sizeof(E) == 4 && D == 128);
  static constexpr bool kRec = kStageQK;
  static constexpr int QKT = kStageQK ? TILE : 0;
  static constexpr int RECS = kRec ? 6 * RECB : 0;
  static constexpr int oT = 0;                          // T, from the forward context
  static constexpr int odP = oT + MAT;                  // dP * D
  static constexpr int oVt = odP + PMAT;                // F(V'; s, j) records
  static constexpr int oDV = oVt + SET;                 // F(dV'; r, j) records, later F(T^T dV'; s, j)
  static constexpr int oG = oDV + SET;                  // G = dV' V'^T (fp32), later dk staging
  static constexpr int oEE = oG + MAT;                  // E + E^T, operand type
  static constexpr int oPDt = oEE + PMAT;               // F(dP*D; s, r) records
  static constexpr int oTt = oPDt + RECS;               // F(T; s, r) records
  static constexpr int oQ = oTt + RECS;                 // staged natural tiles
  static constexpr int oK = oQ + QKT;
  static constexpr int oSm = oK + QKT;
  static constexpr int SMALL = (64 * 2 + NW * 64 * 2 + NW * 2) * 4;
  static constexpr int BASE = oSm + SMALL;
  static constexpr bool kStageDO = BASE + TILE <= 160 * 1024 - 512;
  static constexpr int odO = BASE;
  static constexpr int BYTES = BASE + (kStageDO ? TILE : 0);
  static_assert(BYTES + 128 * 4 <= 160 * 1024, "bwd_grad fits the LDS of a workgroup");
  static_assert(SET >= 2 * NW * 64 * 4, "the dbeta slots fit the dX_u region");
};

template <typename E, int D, bool NORM>
__global__ __launch_bounds__(64 * (D / 16)) void k_bwd_grad(Params p) {
  using S = BwdGradSmem<E, D>;
  constexpr int KB = D / 32, NJ = D / 16, NW = D / 16, LDF = S::LDF, LDE = S::LDE;
  __shared__ __attribute__((aligned(16))) char smem[S::BYTES];
  E* sEE = reinterpret_cast<E*>(smem + S::oEE);
  float* sT = reinterpret_cast<float*>(smem + S::oT);   // T^T: row a holds column a of T
  E* sdP = reinterpret_cast<E*>(smem + S::odP);
  E* sVt = reinterpret_cast<E*>(smem + S::oVt);
  E* sdVt = reinterpret_cast<E*>(smem + S::oDV);
  E* sdXu = reinterpret_cast<E*>(smem + S::oDV);       // after G: F(T^T dV'; s, j) records
  float* sG = reinterpret_cast<float*>(smem + S::oG);   // G^T, G = dV' V'^T
  E* sTt = reinterpret_cast<E*>(smem + S::oTt);        // F(T; s, r) records
  E* sPDt = reinterpret_cast<E*>(smem + S::oPDt);      // F(dP*D; s, r) records
  char* tQ = smem + S::oQ;
  char* tK = smem + S::oK;
  char* tO = smem + S::odO;
  float* s_gam = reinterpret_cast<float*>(smem + S::oSm);
  float* s_beta = s_gam + 64;
  float* s_pg = s_beta + 64;          // [NW][64] dgamma partials
  float* s_pb = s_pg + NW * 64;       // [NW][64] dbeta partials
  float* s_misc = s_pb + NW * 64;     // [NW][2]: sum_s c_s, <h, H'>
  // at the end, in the dX_u records' region (free once the dk phase is done):
  float* s_pq = reinterpret_cast<float*>(smem + S::oDV);   // [NW][64] dbeta partials, quotient form
  float* s_pa = s_pq + NW * 64;                            // [NW][64] partials of ||A_r||^2

  const int ch = blockIdx.x;
  const int H = p.H;
  const int c = ch / H, h = ch - c * H;
  const int4 ct = chunk_info(p, c);
  // the unit one round ahead, for the L2 prefetch below (this unit when none)
  constexpr bool kPrefetch = sizeof(E) == 2 && D == 128;
  const int ua = kPrefetch && p.grad_ahead > 0 && ch + p.grad_ahead < p.NC * H ? ch + p.grad_ahead : ch;
  const int ha = ua % H;
  const int4 cta = kPrefetch ? chunk_info(p, ua / H) : ct;
  const int tok0 = ct.x, L = ct.y;
  const int lane = lane_id(), w = wave_id(), li = lane & 15, lg = lane >> 4;
  const int kw = w >> 1, hw = w & 1;
  const int tid = threadIdx.x;
  constexpr int NT = 64 * NW;
  const E* Q = reinterpret_cast<const E*>(p.q);
  const E* K = reinterpret_cast<const E*>(p.k);
  const E* V = reinterpret_cast<const E*>(p.v);
  const E* dO = reinterpret_cast<const E*>(p.dO);
  const E* Hf = reinterpret_cast<const E*>(p.Hf);
  const E* Vf = reinterpret_cast<const E*>(p.Vf);
  const E* HPf = reinterpret_cast<const E*>(p.HPf);
  const E* dVf = reinterpret_cast<const E*>(p.dVf);
  const float sc = p.scale;
  // q, k and dq, dk: token stride ldq, dk wide; v and dv: token stride ldv, dv
  // wide; dO: contiguous, dv wide.  Columns past a width read as zero.
  const size_t rowstride = (size_t)H * p.vdim;
  const size_t base = ((size_t)tok0 * H + h) * p.vdim;
  const size_t xrow = (size_t)p.ldq;
  const size_t xbase = (size_t)tok0 * xrow + (size_t)h * p.kdim;
  const size_t vrow = (size_t)p.ldv;
  const size_t vbase = (size_t)tok0 * vrow + (size_t)h * p.vdim;

  // natural fragment of row `row`, 32-column block kb, of a tensor `width` wide
  auto gnat = [&](const E* X, size_t xb, size_t xr, int row, int kb, int width) {
    return row < L && 32 * kb < width ? load_frag_row<E>(X + xb + (size_t)row * xr + 32 * kb, lg) : zero_frag<E>();
  };
  __shared__ float s_inv[NORM ? 128 : 1];   // sign-encoded reciprocal norms of the q, k rows
  // natural fragments of Q and K (normalised rows with NORM): from the staged
  // tiles, or from global memory, scaled here
  auto qf = [&](int ab, int kb) {
    if constexpr (S::kStageQK) {
      return tile_frag<E, D>(tQ, ab, kb, li, lg);
    } else {
      const frag_t<E> f = gnat(Q, xbase, xrow, 16 * ab + li, kb, p.kdim);
      if constexpr (NORM) return scale_frag<E>(f, fabsf(s_inv[16 * ab + li]));
      else return f;
    }
  };
  auto kf = [&](int ab, int kb) {
    if constexpr (S::kStageQK) {
      return tile_frag<E, D>(tK, ab, kb, li, lg);
    } else {
      const frag_t<E> f = gnat(K, xbase, xrow, 16 * ab + li, kb, p.kdim);
      if constexpr (NORM) return scale_frag<E>(f, fabsf(s_inv[64 + 16 * ab + li]));
      else return f;
    }
  };
  auto of = [&](int ab, int kb) {
    if constexpr (S::kStageDO) return tile_frag<E, D>(tO, ab, kb, li, lg);
    else return gnat(dO, base, rowstride, 16 * ab + li, kb, p.vdim);
  };
  // fp32 LDS matrix fragments: index rows 16ab.., contraction cols 32kb..
  auto mfrag32 = [&](const float* M, int ab, int kb) {
    const float* row = M + (16 * ab + li) * LDF + 32 * kb;
    return to_frag<float>(*reinterpret_cast<const f32x4*>(row + 4 * lg), *reinterpret_cast<const f32x4*>(row + 16 + 4 * lg));
  };
  // operand-type 64 x 64 matrices (dP*D, E + E^T)
  auto efrag = [&](const E* M, int ab, int kb) { return load_frag_row<E>(M + (16 * ab + li) * LDE + 32 * kb, lg); };
  auto pfragT = [&](int cb, int kb) {
    frag_t<E> t;
#pragma unroll
    for (int e = 0; e < 8; ++e) t[e] = sdP[(32 * kb + kslot(lg, e)) * LDE + 16 * cb + li];
    return t;
  };
  auto lrec = [&](const E* b, int a, int kb) { return load_rec<E>(b + (a * KB + kb) * REC, lane); };
  // records of lower-triangular 64 x 64 matrices read transposed, F(X; s, r)
  // for the six (s-block sb, r-block rkb) with a nonzero entry
  auto tri_idx = [](int sb, int rkb) { return sb < 2 ? 2 * sb + rkb : sb + 2; };
  auto trec = [&](const E* b, int sb, int rkb) { return load_rec<E>(b + tri_idx(sb, rkb) * REC, lane); };
  // half hw of a record: the four elements a 16-column block contributes
  auto store_half = [&](E* rec, f32x4 x) {
    *reinterpret_cast<quad_t<E>*>(rec + 8 * lane + 4 * hw) = to_quad<E>(x);
  };
  // half hw of a record (a quad): the operand of a 16-deep identity
  // transpose, the other half of the contraction being one that is only ever
  // multiplied by zeros
  auto load_half = [&](const E* rec) { return *reinterpret_cast<const quad_t<E>*>(rec + 8 * lane + 4 * hw); };
  // the four elements of a natural fragment that fall in this wave's columns
  auto my4 = [&](f32x8 x) {
    return hw ? f32x4{x[4], x[5], x[6], x[7]} : f32x4{x[0], x[1], x[2], x[3]};
  };
  // Owners of the dA tiles and of the transposed records at 8 waves,
  // balanced by cost: dA tiles of a-block <= 1 take two 32-deep fp32 steps,
  // the others one; a record costs about a third of a one-step tile.  Other
  // wave counts deal round-robin.
  constexpr int DA_OWN8[10] = {0, 1, 2, 3, 4, 5, 6, 7, 3, 4};
  constexpr int TREC_OWN8[12] = {5, 6, 7, 0, 1, 2, 5, 6, 7, 0, 1, 2};
  constexpr int RR4[10] = {0, 1, 2, 3, 0, 1, 2, 3, 0, 1};
  constexpr int RREC4[12] = {3, 2, 1, 0, 3, 2, 1, 0, 3, 2, 1, 0};
  constexpr int MAXT = NW == 8 ? 2 : 3;
  constexpr unsigned long long DA_LIST = NW == 8 ? pack_owned<10, 8, 2>(DA_OWN8) : pack_owned<10, 4, 3>(RR4);
  constexpr unsigned long long TREC_LIST = NW == 8 ? pack_owned<12, 8, 2>(TREC_OWN8) : pack_owned<12, 4, 3>(RREC4);
  static_assert(NW == 8 || NW == 4, "bwd_grad deals its tiles over 4 or 8 waves");

  // ---- setup.  Reads are issued in three groups, each ahead of the phase
  // that waits for it: the staged tiles and T (stored to LDS before the first
  // barrier), the V' and dV' records (transposed after it), and the h and H'
  // record halves with the V rows of dbeta (used after the second).  Issuing
  // all of them at the start measured slower: the reads of a unit stream in
  // at a fixed rate per CU, so the early ones only wait longer.
  frag_t<E> vrec[2], drec[2];      // F(V'; j, s), F(dV'; j, r) of column block w
  quad_t<E> hrec[NJ], hprec[NJ];   // halves of the h and H' records of this wave's i-block
  // V[16 sb + li][32 kw + 16 hw + 4 lg + q], the v_s of this wave's columns:
  // read unconditionally (row and column clamped into the tensor) and zeroed
  // where they fall outside when used, so that no read waits at a branch
  quad_t<E> vq[4];
  auto load_vq = [&]() {
#pragma unroll
    for (int sb = 0; sb < 4; ++sb) {
      const int vr = 16 * sb + li < L ? 16 * sb + li : L - 1;
      const int vc = 32 * kw < p.vdim ? 32 * kw + 16 * hw + 4 * lg : 0;
      vq[sb] = *reinterpret_cast<const quad_t<E>*>(V + vbase + (size_t)vr * vrow + vc);
    }
  };
  {
    const float gv = p.gamma[(size_t)ch * 64 + lane];
    const float bv = lane < L ? p.beta[(size_t)(tok0 + lane) * H + h] : 0.f;
    TileStage<E, D, NT> sq, sk, so;
    const size_t nb = (size_t)tok0 * H + h;   // reciprocal norms of this chunk's rows, stride H
    if constexpr (S::kStageQK) {
      sq.load(Q + xbase, xrow, L, tid, NORM ? p.qinv + nb : nullptr, H, p.kdim);
      sk.load(K + xbase, xrow, L, tid, NORM ? p.kinv + nb : nullptr, H, p.kdim);
    }
    float inv_row = 0.f;   // unstaged: thread r < 128 fetches the scale of q row r or k row r - 64
    if constexpr (NORM && !S::kStageQK) {
      if (tid < 128) {
        const int r = tid & 63;
        inv_row = (tid < 64 ? p.qinv : p.kinv)[nb + (size_t)(r < L ? r : 0) * H];
      }
    }
    if constexpr (S::kStageDO) so.load(dO + base, rowstride, L, tid, nullptr, 0, p.vdim);
    // T = (I + diag(beta) A')^-1 as the forward solved it
    constexpr int TPER = 64 * 16 / NT;
    f32x4 tv[TPER];
#pragma unroll
    for (int k = 0; k < TPER; ++k) {
      // column c, rows 4 r4 .. 4 r4 + 3 (a wave's lanes read whole rows)
      const int e = tid + k * NT, c = e & 63, r4 = e >> 6;
      const float* src = p.Tm + (size_t)ch * 4096 + (4 * r4) * 64 + c;
      tv[k] = f32x4{src[0], src[64], src[128], src[192]};
    }
    // (the decays are written once every read above is in flight)
    if (w == 0) {
      s_gam[lane] = gv;
      s_beta[lane] = bv;
    }
    if constexpr (S::kStageQK) {
      sq.store(tQ, tid);
      sk.store(tK, tid);
      if constexpr (NORM) {
        sq.store_scales(s_inv, tid);
        sk.store_scales(s_inv + 64, tid);
      }
    } else if constexpr (NORM) {
      if (tid < 128) s_inv[tid] = inv_row;
    }
    if constexpr (S::kStageDO) so.store(tO, tid);
#pragma unroll
    for (int k = 0; k < TPER; ++k) {
      const int e = tid + k * NT, c = e & 63, r4 = e >> 6;
      *reinterpret_cast<f32x4*>(&sT[c * LDF + 4 * r4]) = tv[k];
    }
  }
#pragma unroll
  for (int skb = 0; skb < 2; ++skb) {
    vrec[skb] = load_rec<E>(Vf + (((size_t)ch * NJ + w) * 2 + skb) * REC, lane);
    drec[skb] = load_rec<E>(dVf + (((size_t)ch * NJ + w) * 2 + skb) * REC, lane);
  }
  __syncthreads();
  const float gL = s_gam[63];
  const float GL = __expf(gL);
  const frag_t<E> id0 = ident_frag<E>(0, li, lg), id1 = ident_frag<E>(1, li, lg);
  const frag_t<E> idw = hw ? id1 : id0;
  const quad_t<E> idq = ident_quad<E>(li, lg);

  // ---- transposes of this wave's column block of V' and dV' into LDS:
  //      half hw of sVt rec (sb, kw) = F(V'; s, j), of sdVt rec (rb, kw) = F(dV'; r, j)
#pragma unroll
  for (int sbp = 0; sbp < 4; ++sbp) {
    const frag_t<E> idh = (sbp & 1) ? id1 : id0;
    const int skb = sbp >> 1;
    store_half(sVt + (sbp * KB + kw) * REC, mma(vrec[skb], idh, zero4()));
    store_half(sdVt + (sbp * KB + kw) * REC, mma(drec[skb], idh, zero4()));
  }
  // zero the blocks no tile writes: G above the block diagonal (stored
  // transposed: below it) and dP*D above it
  zero_off_blocks<float, false>(sG, LDF, tid, NT);
  zero_off_blocks<E, true>(sdP, LDE, tid, NT);
#pragma unroll
  for (int jb = 0; jb < NJ; ++jb) {
    hrec[jb] = load_half(Hf + (((size_t)ch * NJ + jb) * KB + kw) * REC);
    hprec[jb] = load_half(HPf + (((size_t)ch * NJ + jb) * KB + kw) * REC);
  }
  if constexpr (sizeof(E) == 2) load_vq();
  __syncthreads();

  // Per-token partial sums of dgamma and dbeta stay in registers until the
  // end.  Column-indexed values (token 16 blk + li, equal in the four lane
  // groups) land in lane 16 blk + li; row-indexed values (token 16 blk +
  // 4 lg + q, equal in the 16 lanes of group lg) in lane (li = 4 blk + q, lg).
  float dgc = 0.f, dgr = 0.f, dbc = 0.f, dbr = 0.f;
  float dbq = 0.f, dar = 0.f;   // quotient form of dbeta (column-indexed), ||A_r||^2 (row-indexed)
  auto add_col = [&](float& acc, int blk, float v) { acc += (lg == blk) ? v : 0.f; };
  auto add_row = [&](float& acc, int blk, const float* v4) {
    const int q = li & 3;
    const float x = q == 0 ? v4[0] : (q == 1 ? v4[1] : (q == 2 ? v4[2] : v4[3]));
    acc += ((li >> 2) == blk) ? x : 0.f;
  };

  // ---- dP = dO V'^T, P, and G = dV' V'^T (lower tiles, round-robin):
  //      sdP = dP * D, sG = G, dgamma += rowsum(dP * P) - colsum(dP * P)
#pragma unroll
  for (int k = 0; k < MAXT; ++k) {
    const int t = w + NW * k;
    if (t >= 10) break;
    const int rb = tri_row(t), sb = tri_col(t);
    f32x4 dp = zero4(), qk = zero4(), gt = zero4();
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      const frag_t<E> vs = lrec(sVt, sb, kb);
      dp = mma(of(rb, kb), vs, dp);
      gt = mma(lrec(sdVt, rb, kb), vs, gt);
      qk = mma(qf(rb, kb), kf(sb, kb), qk);
    }
    // lane holds [r = 16rb + 4lg + q][s = 16sb + li]
    const int s_ = 16 * sb + li;
    *reinterpret_cast<f32x4*>(&sG[s_ * LDF + 16 * rb + 4 * lg]) = gt;   // G^T[s][r]
    const float gs = s_gam[s_];
    const f32x4 gr4 = *reinterpret_cast<const f32x4*>(s_gam + 16 * rb + 4 * lg);
    float rs[4], cs = 0.f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int r = 16 * rb + 4 * lg + q;
      const float Dm = s_ <= r ? __expf(gr4[q] - gs) : 0.f;
      const float dpd = dp[q] * Dm;
      sdP[r * LDE + s_] = (E)dpd;
      const float mo = dpd * sc * qk[q];
      rs[q] = mo;
      cs += mo;
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) rs[q] = sum_in_group(rs[q]);
    cs = sum_groups(cs);
    add_row(dgr, rb, rs);
    add_col(dgc, sb, -cs);
  }

  // ---- transposes of h and H' for this wave's i-block
  frag_t<E> hT[KB], hpT[KB];   // F(h; i, j), F(H'; i, j) for i-block w
  {
    float hh = 0.f;
#pragma unroll
    for (int jkb = 0; jkb < KB; ++jkb) {
      const f32x4 a0 = mma16(hrec[2 * jkb], idq, zero4());
      const f32x4 a1 = mma16(hrec[2 * jkb + 1], idq, zero4());
      hT[jkb] = to_frag<E>(a0, a1);
      const f32x4 b0 = mma16(hprec[2 * jkb], idq, zero4());
      const f32x4 b1 = mma16(hprec[2 * jkb + 1], idq, zero4());
      hpT[jkb] = to_frag<E>(b0, b1);
#pragma unroll
      for (int q = 0; q < 4; ++q) hh += a0[q] * b0[q] + a1[q] * b1[q];
    }
    hh = sum_in_group(sum_groups(hh));
    if (lane == 0) s_misc[2 * w + 1] = hh;
  }
  __syncthreads();

  // ---- dA = strict_lower(-T^T G); dbeta, dgamma terms of A; E + E^T -> sEE
#pragma unroll
  for (int k = 0; k < MAXT; ++k) {
    const int t = owned_item(DA_LIST, w, MAXT, k);
    if (t == 15) break;
    const int ab = tri_row(t), bb = tri_col(t);
    // every operand read first, then the products (one LDS latency per tile)
    f32x8 tf[2], gf[2];
    frag_t<E> ka[KB], kb_[KB];
    const bool two = ab <= 1;   // T[r][a] = 0 for r < a: the first 32-block of r only for a-block <= 1
#pragma unroll
    for (int rkb = 0; rkb < 2; ++rkb) {
      tf[rkb] = (rkb == 1 || two) ? mfrag32(sT, ab, rkb) : f32x8{};
      gf[rkb] = (rkb == 1 || two) ? mfrag32(sG, bb, rkb) : f32x8{};
    }
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      ka[kb] = kf(ab, kb);
      kb_[kb] = kf(bb, kb);
    }
    __builtin_amdgcn_sched_barrier(0);
    f32x4 acc = zero4(), kk = zero4();
    if (two) acc = mma(tf[0], gf[0], acc);
    acc = mma(tf[1], gf[1], acc);
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) kk = mma(ka[kb], kb_[kb], kk);
    // lane holds -dA[a = 16ab + 4lg + q][b = 16bb + li] and (K K^T)[a][b]
    const int b = 16 * bb + li;
    const float gb = s_gam[b];
    const f32x4 ga4 = *reinterpret_cast<const f32x4*>(s_gam + 16 * ab + 4 * lg);
    const f32x4 be4 = *reinterpret_cast<const f32x4*>(s_beta + 16 * ab + 4 * lg);
    float rs_b[4], rs_a[4], cs = 0.f;
    f32x4 ev;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int a = 16 * ab + 4 * lg + q;
      float da = 0.f, ap = 0.f, Dm = 0.f;
      if (ab > bb || a > b) {
        da = -acc[q];
        Dm = __expf(ga4[q] - gb);
        ap = kk[q] * Dm;   // A'[a][b]
      }
      rs_b[q] = da * ap;
      rs_a[q] = ap * ap;
      cs += da * be4[q] * ap;
      ev[q] = da * be4[q] * Dm;   // E[a][b]; zero on and above the diagonal
    }
    // E + E^T into sEE: E[a][b] at (a, b) and at (b, a).  Off the block
    // diagonal the mirrored values of a lane are four consecutive entries of
    // row b; in a diagonal block every entry of the block is written once,
    // by the lane holding it or its mirror.
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int a = 16 * ab + 4 * lg + q;
      if (ab > bb || a > b) sEE[a * LDE + b] = (E)ev[q];
      else if (a == b) sEE[a * LDE + a] = (E)0.f;
    }
    if (ab > bb) {
      *reinterpret_cast<quad_t<E>*>(sEE + b * LDE + 16 * ab + 4 * lg) = to_quad<E>(ev);
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int a = 16 * ab + 4 * lg + q;
        if (a > b) sEE[b * LDE + a] = (E)ev[q];
      }
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      rs_b[q] = sum_in_group(rs_b[q]);
      rs_a[q] = sum_in_group(rs_a[q]);
    }
    // the dgamma row term is beta_a times the dbeta one; ||A_a||^2 = beta_a^2 sum_b A'^2
    float rs_g[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      rs_g[q] = be4[q] * rs_b[q];
      rs_a[q] *= be4[q] * be4[q];
    }
    cs = sum_groups(cs);
    add_row(dbr, ab, rs_b);
    add_row(dgr, ab, rs_g);
    add_row(dar, ab, rs_a);
    add_col(dgc, bb, -cs);
  }
  // transposed records of T and dP*D for the output phase, once per workgroup
#pragma unroll
  for (int j = 0; j < (S::kRec ? MAXT : 0); ++j) {
    const int k = owned_item(TREC_LIST, w, MAXT, j);
    if (k == 15) break;
    const int kk = k < 6 ? k : k - 6;
    const int sb = kk < 4 ? kk >> 1 : kk - 2, rkb = kk < 4 ? kk & 1 : 1;
    frag_t<E> x;
    if (k < 6) {
      x = f32_to_frag<E>(mfrag32(sT, sb, rkb));
      store_rec<E>(sTt + kk * REC, lane, x);
    } else {
      x = pfragT(sb, rkb);
      store_rec<E>(sPDt + kk * REC, lane, x);
    }
  }
  // (in fp32 the V rows are read here: held across the dP and dA phases,
  // their 16 registers would spill)
  if constexpr (sizeof(E) == 4) load_vq();
  __syncthreads();
  // L2 prefetch for the unit one round ahead (bf16, d = 128).  With one
  // workgroup per CU the units of a round read at the same time and then
  // compute with HBM idle; the unit `grad_ahead` further on (a multiple of 8,
  // so on this XCD) runs next round, and the lines of its first phase (Q, K
  // and dO rows and T: 512 lines of 128 bytes, one per thread) are touched
  // now, one 4-byte read each.  The reads are unconditional (all on one line
  // of this unit's T when none is ahead): behind a branch, the compiler's
  // waits for this unit's reads would also wait for them.  Their value is
  // consumed before this unit's first store, as waits count stores too.
  // They go out here, after the dA phase: issued at the second barrier the
  // backward measured about 1 us slower, after the dX_u barrier slower still.
  int pf = 0;
  if constexpr (kPrefetch) {
    static_assert(NT == 512, "one line per thread");
    const int rr = (tid & 127) >> 1, part = tid & 1;
    const int row = rr < cta.y ? rr : 0;
    const size_t xa = (size_t)cta.x * xrow + (size_t)ha * p.kdim;
    const size_t oa = ((size_t)cta.x * H + ha) * p.vdim;
    const E* a;
    if (tid < 128) a = Q + xa + (size_t)row * xrow + (64 * part < p.kdim ? 64 * part : 0);
    else if (tid < 256) a = K + xa + (size_t)row * xrow + (64 * part < p.kdim ? 64 * part : 0);
    else if (tid < 384) a = dO + oa + (size_t)row * rowstride + (64 * part < p.vdim ? 64 * part : 0);
    else a = reinterpret_cast<const E*>(p.Tm + (size_t)ua * 4096 + 32 * (tid - 384));
    if (ua == ch) a = reinterpret_cast<const E*>(p.Tm + (size_t)ch * 4096);   // none ahead: one line
    pf = *reinterpret_cast<const int*>(a);
  }

  // ---- per-wave outputs.  With in-operator normalisation the gradients just
  // computed are those of the normalised rows, y = x / ||x||; their per-row
  // dots y . dy over all D columns are gathered in LDS (G's region is free
  // now) and dx = (dy - y (y . dy)) / ||x|| is formed after a barrier: dq's
  // right after its products, dk's at the end.
  constexpr bool norm = NORM;
  float* s_qd = sG;             // [64][NW] partial q . dq
  float* s_kd = sG + NW * 64;   // [64][NW] partial k . dk
  // dq, dk, dv leave through LDS: each wave holds 16 columns of a row (32
  // bytes in bf16), so its own stores would write partial lines; staged, the
  // rows go out whole, 16 bytes a lane, after the last barrier.  Staging
  // rows are unpadded, their 16-byte pieces XOR-swizzled by the row so that
  // the column-block writes of a wave fall in distinct banks.  Regions: dq in
  // T's (free after the records are made); dk in G's (free after the dA
  // phase) or, normalised, in Q's tile (free after the last barrier); dv in
  // K's tile.
  constexpr int RB = D * (int)sizeof(E);   // bytes of a staged row
  constexpr int PPR = RB / 16;             // 16-byte pieces per row
  constexpr bool kStageOut = S::kStageQK;
  static_assert(!kStageOut || (64 * RB <= S::MAT && 64 * RB <= S::TILE), "a staged output tile fits its region");
  // staging regions, or (unstaged) the gradient tensors themselves
  char* stq = kStageOut ? reinterpret_cast<char*>(sT) : reinterpret_cast<char*>(p.dq);
  char* stk = kStageOut ? (norm ? tQ : reinterpret_cast<char*>(sG)) : reinterpret_cast<char*>(p.dk);
  char* stv = kStageOut ? tK : reinterpret_cast<char*>(p.dv);
  // columns 16 w + 4 lg .. + 3 of row r (this lane's four values) into a
  // staging tile, or straight to row r of the gradient (rows < L and columns
  // inside its width only); is_v: the tensor is dv (else dq or dk)
  auto stage4 = [&](char* st, int r, f32x4 x, bool is_v) {
    const int byte = (16 * w + 4 * lg) * (int)sizeof(E);
    if constexpr (kStageOut) {
      const int pc = (byte >> 4) ^ (r % PPR);
      *reinterpret_cast<quad_t<E>*>(st + r * RB + 16 * pc + (byte & 15)) = to_quad<E>(x);
    } else {
      const size_t row0 = is_v ? vbase + (size_t)r * vrow : xbase + (size_t)r * xrow;
      if (r < L && 16 * w < (is_v ? p.vdim : p.kdim))
        store_quad_nt<E>(reinterpret_cast<E*>(st + row0 * sizeof(E) + byte), x);
    }
  };
  f32x4 dqh[4], dkh[4], qn4[4], kn4[4];
  // dx for rows 16 rb + li of this wave's columns (rows above the floor:
  // (dy - y (y . dy)) / ||x||; below it: dy / floor), into a staging tile
  auto norm_out = [&](const f32x4 (&dy)[4], const f32x4 (&yn)[4], const float* part, const float* iv, char* dst) {
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      const int r = 16 * rb + li;
      float yd = 0.f;
#pragma unroll
      for (int w4 = 0; w4 < NW; w4 += 4) {
        const f32x4 a = *reinterpret_cast<const f32x4*>(part + r * NW + w4);
#pragma unroll
        for (int q = 0; q < 4; ++q) yd += a[q];
      }
      const float ir = iv[r];
      f32x4 o;
#pragma unroll
      for (int q = 0; q < 4; ++q) o[q] = ir > 0.f ? (dy[rb][q] - yn[rb][q] * yd) * ir : -dy[rb][q] * ir;
      stage4(dst, r, o, false);
    }
  };
  // F(T; s, r) and F(dP*D; s, r): from their records, or read transposed
  auto tt = [&](int sb, int rkb) {
    if constexpr (S::kRec) return trec(sTt, sb, rkb);
    else return f32_to_frag<E>(mfrag32(sT, sb, rkb));
  };
  auto pdt = [&](int sb, int rkb) {
    if constexpr (S::kRec) return trec(sPDt, sb, rkb);
    else return pfragT(sb, rkb);
  };
  // dX_u = T^T dV' for this wave's j-block, first: dV = diag(beta) dX_u, the
  // dbeta terms v_s . dX_u[s] (sum) and V'_s . dX_u[s] / beta_s (quotient), and
  // its records (all waves' blocks) give dX_w = T^T dW = -dX_u h^T in the dk phase.
  // Accumulator sb holds dX_u^T[j = 16w + 4lg + q][s = 16sb + li], which is
  // half hw of the record F(dX_u; s, j) (sb, kw); the same half of the record
  // F(V'; s, j) holds V' at the same (s, j).
  f32x4 dvo[4];
  {
    f32x4 acc[4];
#pragma unroll
    for (int sb = 0; sb < 4; ++sb) acc[sb] = zero4();
#pragma unroll
    for (int rkb = 0; rkb < 2; ++rkb)
#pragma unroll
      for (int sb = 0; sb < 4; ++sb) {
        if (32 * rkb + 31 < 16 * sb) continue;
        acc[sb] = mma(drec[rkb], tt(sb, rkb), acc[sb]);
      }
#pragma unroll
    for (int sb = 0; sb < 4; ++sb) {
      const int s_ = 16 * sb + li;
      const float bs = s_beta[s_];
      const f32x4 vv = s_ < L && 32 * kw < p.vdim ? quad_to_f32<E>(vq[sb]) : zero4();
      const f32x4 vp = my4(frag_to_f32<E>(lrec(sVt, sb, kw)));
      float dot = 0.f, dqt = 0.f;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        dot += vv[q] * acc[sb][q];
        dqt += vp[q] * acc[sb][q];
      }
      dot = sum_groups(dot);
      dqt = sum_groups(dqt);
      add_col(dbc, sb, dot);
      add_col(dbq, sb, bs != 0.f ? __fdividef(dqt, bs) : 0.f);
      dvo[sb] = scale4(acc[sb], bs);
      store_half(sdXu + (sb * KB + kw) * REC, acc[sb]);
    }
  }
  // K and Q transposes for this wave's i-block: F(K; i, s), F(Q; i, r)
  frag_t<E> kT[2], qT[2];
  {
    f32x4 tk[4], tq[4];
#pragma unroll
    for (int sb = 0; sb < 4; ++sb) {
      tk[sb] = mma(kf(sb, kw), idw, zero4());
      tq[sb] = mma(qf(sb, kw), idw, zero4());
    }
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2) {
      kT[kb2] = to_frag<E>(tk[2 * kb2], tk[2 * kb2 + 1]);
      qT[kb2] = to_frag<E>(tq[2 * kb2], tq[2 * kb2 + 1]);
    }
  }
  __syncthreads();   // every block of dX_u is in sdXu

  // dQ^T[i][r] = scale (Gam_r sum_j h[i][j] dO[r][j] + sum_s K[s][i] dPD[r][s])
  {
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      const int r = 16 * rb + li;
      f32x4 t1 = zero4(), aq = zero4();
#pragma unroll
      for (int jkb = 0; jkb < KB; ++jkb) t1 = mma(hT[jkb], of(rb, jkb), t1);
#pragma unroll
      for (int skb = 0; skb < 2; ++skb) {
        if (32 * skb > 16 * rb + 15) continue;
        aq = mma(kT[skb], efrag(sdP, rb, skb), aq);
      }
      // dgamma(r) += Gam_r sum_i (scale Q[r][i]) t1[i][r]
      const f32x4 qn = my4(frag_to_f32<E>(qf(rb, kw)));
      float dot = 0.f;
#pragma unroll
      for (int q = 0; q < 4; ++q) dot += qn[q] * t1[q];
      dot = sum_groups(dot);
      const float Gr = __expf(s_gam[r]);
      add_col(dgc, rb, sc * Gr * dot);
      f32x4 acc;
#pragma unroll
      for (int q = 0; q < 4; ++q) acc[q] = sc * (Gr * t1[q] + aq[q]);
      if constexpr (norm) {
        float yd = 0.f;
#pragma unroll
        for (int q = 0; q < 4; ++q) yd += qn[q] * acc[q];
        yd = sum_groups(yd);
        if (lg == 0) s_qd[r * NW + w] = yd;
        dqh[rb] = acc;
        qn4[rb] = qn;
      } else {
        stage4(stq, r, acc, false);
      }
    }
    if constexpr (norm) {
      __syncthreads();
      norm_out(dqh, qn4, s_qd, s_inv, stq);
    }
  }

  // dK^T[i][s] = scale sum_r Q[r][i] dPD[r][s] + exp(gL - g_s) sum_j H'[i][j] V'[s][j]
  //            + beta_s Gam_s dX_w[s][i] + sum_r K[r][i] (E + E^T)[s][r],
  // dX_w[s][i] = -sum_j dX_u[s][j] h[i][j]
  {
    f32x4 ta[4], tb[4], tc[4], td[4];
#pragma unroll
    for (int sb = 0; sb < 4; ++sb) {
      ta[sb] = zero4();
      tb[sb] = zero4();
      tc[sb] = zero4();
      td[sb] = zero4();
    }
#pragma unroll
    for (int jkb = 0; jkb < KB; ++jkb)
#pragma unroll
      for (int sb = 0; sb < 4; ++sb) {
        tb[sb] = mma(hpT[jkb], lrec(sVt, sb, jkb), tb[sb]);
        tc[sb] = mma(hT[jkb], lrec(sdXu, sb, jkb), tc[sb]);
      }
#pragma unroll
    for (int sb = 0; sb < 4; ++sb) tc[sb] = -tc[sb];
#pragma unroll
    for (int rkb = 0; rkb < 2; ++rkb)
#pragma unroll
      for (int sb = 0; sb < 4; ++sb) {
        td[sb] = mma(kT[rkb], efrag(sEE, sb, rkb), td[sb]);
        if (32 * rkb + 31 < 16 * sb) continue;  // dPD[r][s] vanishes for r < s
        ta[sb] = mma(qT[rkb], pdt(sb, rkb), ta[sb]);
      }
    float csum = 0.f;
#pragma unroll
    for (int sb = 0; sb < 4; ++sb) {
      const int s_ = 16 * sb + li;
      const float gs = s_gam[s_], Gs = __expf(gs), bs = s_beta[s_], ks = __expf(gL - gs);
      // per-s dots with k_s over this wave's i-block: c_s and k_s . dXw_s
      const f32x4 kn = my4(frag_to_f32<E>(kf(sb, kw)));
      float dc = 0.f, dx = 0.f;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        dc += kn[q] * tb[sb][q];
        dx += kn[q] * tc[sb][q];
      }
      dc = sum_groups(dc) * ks;   // c_s (partial)
      dx = sum_groups(dx);
      add_col(dgc, sb, -dc + bs * Gs * dx);
      add_col(dbc, sb, Gs * dx);
      csum += (lg == 0) ? dc : 0.f;
      f32x4 acc;
#pragma unroll
      for (int q = 0; q < 4; ++q) acc[q] = sc * ta[sb][q] + ks * tb[sb][q] + bs * Gs * tc[sb][q] + td[sb][q];
      if constexpr (norm) {
        float yd = 0.f;
#pragma unroll
        for (int q = 0; q < 4; ++q) yd += kn[q] * acc[q];
        yd = sum_groups(yd);
        if (lg == 0) s_kd[s_ * NW + w] = yd;
        dkh[sb] = acc;
        kn4[sb] = kn;
      } else {
        stage4(stk, s_, acc, false);
      }
    }
    csum = sum_in_group(csum);
    if (lane == 0) s_misc[2 * w] = csum;
  }

  // the prefetch's value, long arrived, before any store of this unit
  if constexpr (kPrefetch) asm volatile("" ::"v"(pf));
  {
    // this wave's slots: the row-indexed sums are stored, the column-indexed
    // ones added (one wave's LDS accesses complete in order)
    float* pg = s_pg + w * 64;
    float* pb = s_pb + w * 64;
    const int tr = 16 * (li >> 2) + 4 * lg + (li & 3);
    pg[tr] = dgr;
    pb[tr] = dbr;
    pg[lane] += dgc;
    pb[lane] += dbc;
  }
  __syncthreads();
  {
    const int tr = 16 * (li >> 2) + 4 * lg + (li & 3);
    s_pa[w * 64 + tr] = dar;
    s_pq[w * 64 + lane] = dbq;
  }

  if constexpr (norm) norm_out(dkh, kn4, s_kd, s_inv + 64, stk);
#pragma unroll
  for (int sb = 0; sb < 4; ++sb) stage4(stv, 16 * sb + li, dvo[sb], true);
  __syncthreads();
  // whole rows of dq, dk, dv, 16 bytes a lane, non-temporal: another kernel
  // reads them next, and a step's 48 MB of them left dirty in the caches
  // would be written back in the middle of later kernels' reads
  static_assert((64 * PPR) % NT == 0, "the staged rows divide over the threads");
  const int ppq = p.kdim * (int)sizeof(E) / 16, ppv = p.vdim * (int)sizeof(E) / 16;   // pieces of a row that exist
#pragma unroll
  for (int e0 = 0; e0 < (kStageOut ? 64 * PPR : 0); e0 += NT) {
    const int e = e0 + tid, r = e / PPR, pc = e - r * PPR;
    if (r < L) {
      const int off = r * RB + 16 * (pc ^ (r % PPR));
      if (pc < ppq) {
        const size_t dst = (xbase + (size_t)r * xrow) * sizeof(E) + 16 * (size_t)pc;
        __builtin_nontemporal_store(*reinterpret_cast<const i32x4*>(stq + off), reinterpret_cast<i32x4*>(reinterpret_cast<char*>(p.dq) + dst));
        __builtin_nontemporal_store(*reinterpret_cast<const i32x4*>(stk + off), reinterpret_cast<i32x4*>(reinterpret_cast<char*>(p.dk) + dst));
      }
      if (pc < ppv) {
        const size_t dst = (vbase + (size_t)r * vrow) * sizeof(E) + 16 * (size_t)pc;
        __builtin_nontemporal_store(*reinterpret_cast<const i32x4*>(stv + off), reinterpret_cast<i32x4*>(reinterpret_cast<char*>(p.dv) + dst));
      }
    }
  }

  // ---- dgamma -> dg (reverse chunk-local cumsum), dbeta
  if (w == 0) {
    const int r = lane;
    float dgam = 0.f, db = 0.f, dbt = 0.f, an = 0.f, ctot = 0.f, hh = 0.f;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) {
      dgam += s_pg[ww * 64 + r];
      db += s_pb[ww * 64 + r];
      dbt += s_pq[ww * 64 + r];
      an += s_pa[ww * 64 + r];
      ctot += s_misc[2 * ww];
      hh += s_misc[2 * ww + 1];
    }
    if (r == L - 1) dgam += ctot + GL * hh;
    if (an > 1.f) db = dbt;
    if (r >= L) dgam = 0.f;
    // reverse inclusive scan over lanes
    float x = dgam;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float tt = __shfl_down(x, off, 64);
      if (r + off < 64) x += tt;
    }
    if (r < L) {
      p.dg[(size_t)(tok0 + r) * H + h] = x;
      p.dbeta[(size_t)(tok0 + r) * H + h] = db;
    }
  }
}

// --------------------------------------------------------------------------
template <typename E, int D>
static hipError_t bwd_prep_t(const Params& p, hipStream_t s) {
  if (p.NC == 0) return hipSuccess;
  Params a = p;
  void* args[] = {&a};
  return hipLaunchKernel(p.qk_l2norm ? (const void*)k_bwd_prep<E, D, true> : (const void*)k_bwd_prep<E, D, false>, dim3(p.NC * p.H), dim3(64 * (D / 32)), args, 0, s);
}
template <typename E, int D>
static hipError_t bwd_state_t(const Params& p, hipStream_t s) {
  if (p.N * p.H == 0) return hipSuccess;
  Params a = p;
  void* args[] = {&a};
  // two column blocks per workgroup (a grid past one round; always with rotated
  // reads) where the ring's slots for them fit the LDS
  if constexpr (BwdRing<E, D, 2>::FITS) {
    if (p.state_cpw == 2)
      return hipLaunchKernel((const void*)k_bwd_state<E, D, true, 2>, dim3(state_grid(p.N * p.H, D, 2)),
                             dim3(64 * BwdRing<E, D, 2>::WAVES), args, 0, s);
  }
  return hipLaunchKernel(p.dma_rot ? (const void*)k_bwd_state<E, D, true, 1> : (const void*)k_bwd_state<E, D, false, 1>,
                         dim3(state_grid(p.N * p.H, D)), dim3(64 * BwdRing<E, D, 1>::WAVES), args, 0, s);
}
template <typename E, int D>
static hipError_t bwd_grad_t(const Params& p, hipStream_t s) {
  if (p.NC == 0) return hipSuccess;
  Params a = p;
  void* args[] = {&a};
  return hipLaunchKernel(p.qk_l2norm ? (const void*)k_bwd_grad<E, D, true> : (const void*)k_bwd_grad<E, D, false>, dim3(p.NC * p.H), dim3(64 * (D / 16)), args, 0, s);
}

#define GDN_BWD_DISPATCH(fn, ...)                                    \
  do {                                                               \
    if (is_bf16) {                                                   \
      if (D == 64) return fn<bf16, 64>(__VA_ARGS__);                 \
      if (D == 128) return fn<bf16, 128>(__VA_ARGS__);               \
    } else {                                                         \
      if (D == 64) return fn<float, 64>(__VA_ARGS__);                \
      if (D == 128) return fn<float, 128>(__VA_ARGS__);              \
    }                                                                \
    return hipErrorInvalidValue;                                     \
  } while (0)

hipError_t launch_bwd_prep(const Params& p, int D, bool is_bf16, hipStream_t s) { GDN_BWD_DISPATCH(bwd_prep_t, p, s); }
hipError_t launch_bwd_state(const Params& p, int D, bool is_bf16, hipStream_t s) { GDN_BWD_DISPATCH(bwd_state_t, p, s); }
hipError_t launch_bwd_grad(const Params& p, int D, bool is_bf16, hipStream_t s) { GDN_BWD_DISPATCH(bwd_grad_t, p, s); }

}  // namespace gdn
