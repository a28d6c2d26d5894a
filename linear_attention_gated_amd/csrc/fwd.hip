// fwd.hip -- chunk planner and the forward kernels of the gated delta rule.
//
// Chunked form (per sequence and head; chunks of 64 tokens restart at each
// sequence start; rows r, s of a chunk; h = S^T is d_k x d_v):
//   gamma_r = sum_{s<=r} g_s,  Gam = exp(gamma),  D_rs = exp(gamma_r - gamma_s) (s <= r)
//   A  = strict_lower(diag(beta) (K K^T) * D),   T = (I + A)^-1
//   W  = T diag(beta Gam) K,    U = T diag(beta) V
//   V' = U - W h
//   O  = scale [diag(Gam) Q h + ((Q K^T) * D) V']
//   h' = exp(gamma_L) h + Kt^T V',   Kt = diag(exp(gamma_L - gamma)) K
// This is the decomposition of the native kernel family in the XTuner /
// Ascend 910C article (section 3.1.2, Fig. 7 and Fig. 8): an intra-chunk
// triangular solve (solve_tril), a forward state update across chunks and an
// output step; the equations are derived from the token recurrence.
#include "frag.h"
#include "gdn_internal.h"
#include "ring.h"
#include "tri.h"

namespace gdn {

// --------------------------------------------------------------------------
// Planner: chunk table and sequence table from cu_seqlens (packed input only).
// One workgroup: a scan over sequences for the first-chunk offsets, then a
// binary search per chunk.
__global__ __launch_bounds__(1024) void k_plan(Params p) {
  __shared__ int s_scan[1024];
  __shared__ int s_carry;
  const int tid = threadIdx.x;
  if (tid == 0) s_carry = 0;
  __syncthreads();
  for (int base = 0; base < p.N; base += 1024) {
    const int n = base + tid;
    int t0 = 0, len = 0, nc = 0;
    if (n < p.N) {
      if (p.cu) {
        t0 = p.cu[n];
        len = p.cu[n + 1] - t0;
      } else {
        t0 = n * p.dense_T;
        len = p.dense_T;
      }
      nc = len > 0 ? (len + CHUNK - 1) / CHUNK : 0;
    }
    s_scan[tid] = nc;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {
      const int add = tid >= off ? s_scan[tid - off] : 0;
      __syncthreads();
      s_scan[tid] += add;
      __syncthreads();
    }
    const int incl = s_scan[tid];
    if (n < p.N) {
      // clamp to the chunk count and token count the host planned for, so a
      // device cu_seqlens that differs from the host copy cannot send any
      // kernel outside its buffers
      const int cs = min(s_carry + incl - nc, p.NC);
      const int ts = min(max(t0, 0), p.total_tokens);
      p.seq_tab[n] = make_int4(cs, min(nc, p.NC - cs), ts, min(max(len, 0), p.total_tokens - ts));
    }
    __syncthreads();
    if (tid == 1023) s_carry += incl;
    __syncthreads();
  }
  __threadfence();
  __syncthreads();
  for (int c = tid; c < p.NC; c += 1024) {
    int lo = 0, hi = p.N - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (p.seq_tab[mid].x <= c) lo = mid; else hi = mid - 1;
    }
    const int4 s = p.seq_tab[lo];
    const int j = c - s.x;
    // t0 stays a valid token even for a chunk clamped to length 0, so that
    // row reads clamped to the chunk's rows never leave the tensors
    const int t0 = min(s.z + CHUNK * j, p.total_tokens - 1);
    const int len = max(0, min(min(CHUNK, s.w - CHUNK * j), p.total_tokens - t0));
    p.chunk_tab[c] = make_int4(t0, len, lo, j);
  }
}

// --------------------------------------------------------------------------
// --------------------------------------------------------------------------
// K1: per (chunk, head): gamma, A, T = (I + A)^-1 (also stored for the
// backward), and the fragment-native operands of the state pass: -W, Kt^T,
// U.  D/32 waves; wave w owns feature columns [32w, 32w + 32).
template <typename E, int D, bool NORM>
__global__ __launch_bounds__(64 * (D / 32)) __attribute__((amdgpu_waves_per_eu(sizeof(E) == 2 ? 4 : 1))) void k_fwd_prep(Params p) {
  constexpr int NW = D / 32;
  constexpr int KB = D / 32;
  constexpr int LDA = 68;
  __shared__ __attribute__((aligned(16))) float sA[64 * LDA];
  __shared__ __attribute__((aligned(16))) float sT[64 * LDA];
  __shared__ float s_gam[64], s_beta[64], s_ks[64];

  const int ch = blockIdx.x;
  const int H = p.H;
  const int c = ch / H, h = ch - c * H;
  const int4 ct = chunk_info(p, c);
  const int tok0 = ct.x, L = ct.y;
  const int lane = lane_id(), w = wave_id(), li = lane & 15, lg = lane >> 4;
  const int tid = threadIdx.x;
  const E* K = reinterpret_cast<const E*>(p.k);
  const E* V = reinterpret_cast<const E*>(p.v);

  // natural key fragments F(K; s, i) for all row blocks, and this wave's
  // value columns (used after the solve; their reads overlap it).  Where the
  // tiles fit the solver's buffers (not yet in use), K and V are staged
  // through LDS with 16-byte row-contiguous reads; otherwise each fragment
  // is read from global memory directly.
  // (raw keys: with normalisation the Gram tiles take both rows' reciprocal
  // norms, and this wave's key columns are scaled once selected)
  constexpr bool kStage = NatTile<E, D>::BYTES <= 64 * LDA * 4;
  frag_t<E> kf[4][KB], vfw[4];
  TileStage<E, D, 64 * NW> sk, sv;
  // (keys dk and values dv wide, zero past that: the records below are D wide)
  const size_t kbase = (size_t)tok0 * p.ldq + (size_t)h * p.kdim, vbase = (size_t)tok0 * p.ldv + (size_t)h * p.vdim;
  if constexpr (kStage) {
    sk.load(K + kbase, (size_t)p.ldq, L, tid, nullptr, 0, p.kdim);
    sv.load(V + vbase, (size_t)p.ldv, L, tid, nullptr, 0, p.vdim);
  } else {
#pragma unroll
    for (int sb = 0; sb < 4; ++sb) {
      const int row = 16 * sb + li;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
        kf[sb][kb] = row < L && 32 * kb < p.kdim ? load_frag_row<E>(K + kbase + (size_t)row * p.ldq + 32 * kb, lg)
                                               : zero_frag<E>();
      vfw[sb] = row < L && 32 * w < p.vdim ? load_frag_row<E>(V + vbase + (size_t)row * p.ldv + 32 * w, lg)
                                         : zero_frag<E>();
    }
  }
  // chunk-local cumulative log decay (read after the key and value reads are
  // in flight); padded rows get g = 0, beta = 0
  float gv = 0.f, bv = 0.f;
  if (lane < L) {
    gv = p.g[(size_t)(tok0 + lane) * H + h];
    bv = p.beta[(size_t)(tok0 + lane) * H + h];
  }
  const float gam = wave_incl_scan(gv, lane);
  if (w == 0) {
    s_gam[lane] = gam;
    s_beta[lane] = bv;
    p.gamma[(size_t)ch * 64 + lane] = gam;
  }
  if constexpr (kStage) {
    char* tK = reinterpret_cast<char*>(sT);
    char* tV = reinterpret_cast<char*>(sA);
    sk.store(tK, tid);
    sv.store(tV, tid);
    __syncthreads();
#pragma unroll
    for (int sb = 0; sb < 4; ++sb) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) kf[sb][kb] = tile_frag<E, D>(tK, sb, kb, li, lg);
      vfw[sb] = tile_frag<E, D>(tV, sb, w, li, lg);
    }
    // (the barrier below also keeps sA and sT from being rewritten while
    // other waves still read their fragments)
  }
  if constexpr (NORM) {
    // sign-encoded reciprocal key norms; every wave holds whole rows, wave 0
    // publishes them (LDS, and the context for the later passes)
#pragma unroll
    for (int sb = 0; sb < 4; ++sb) {
      float ss = 0.f;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const f32x8 f = frag_to_f32<E>(kf[sb][kb]);
#pragma unroll
        for (int e = 0; e < 8; ++e) ss += f[e] * f[e];
      }
      ss = sum_groups(ss);
      const float n = sqrtf(ss);
      const float iv = n > 1e-12f ? 1.f / n : -1.f / 1e-12f;
      const int row = 16 * sb + li;
      if (w == 0 && lg == 0) {
        s_ks[row] = fabsf(iv);
        if (row < L) p.kinv[(size_t)(tok0 + row) * H + h] = iv;
      }
    }
  }
  __syncthreads();

  // A = strict_lower(diag(beta) K K^T * D): ten lower tiles, round-robin over waves
  {
    constexpr int TR[10] = {0, 1, 1, 2, 2, 2, 3, 3, 3, 3};
    constexpr int TS[10] = {0, 0, 1, 0, 1, 2, 0, 1, 2, 3};
#pragma unroll
    for (int t = 0; t < 10; ++t) {
      if (t % NW != w) continue;
      const int rr = TR[t], sc = TS[t];
      f32x4 acc = zero4();
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) acc = mma(kf[sc][kb], kf[rr][kb], acc);
      // lane holds G[r = 16rr + li][s = 16sc + 4lg + q]
      const int r = 16 * rr + li;
      const float gr = s_gam[r], br = NORM ? s_beta[r] * s_ks[r] : s_beta[r];
      float4 out;
      float* po = reinterpret_cast<float*>(&out);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int s = 16 * sc + 4 * lg + q;
        const float a = br * acc[q] * __expf(gr - s_gam[s]);
        po[q] = s < r ? (NORM ? a * s_ks[s] : a) : 0.f;
      }
      *reinterpret_cast<float4*>(&sA[r * LDA + 16 * sc + 4 * lg]) = out;
    }
  }
  // this wave's key columns F(K; s, i in 32w..32w+31)
  frag_t<E> kw[4];
#pragma unroll
  for (int sb = 0; sb < 4; ++sb) {
    kw[sb] = kf[sb][0];
#pragma unroll
    for (int kb = 1; kb < KB; ++kb)
      if (kb == w) kw[sb] = kf[sb][kb];
    if constexpr (NORM) kw[sb] = scale_frag<E>(kw[sb], s_ks[16 * sb + li]);
  }
  __syncthreads();

  // T = (I + A)^-1 (ends with a barrier); kept for the backward, which is
  // the next to read it: stored non-temporal, so that it does not sit dirty
  // in the caches until then
  tri_inverse64(sA, nullptr, sT, LDA, NW);
  for (int e = tid; e < 64 * 16; e += 64 * NW) {
    const int r = e >> 4, c4 = e & 15;
    __builtin_nontemporal_store(*reinterpret_cast<const f32x4*>(&sT[r * LDA + 4 * c4]),
                                reinterpret_cast<f32x4*>(p.Tm + (size_t)ch * 4096 + r * 64 + 4 * c4));
  }

  // T fragments F(T; r, s), read where used (lower triangular: (rb <= 1, skb = 1) is zero)
  auto tfrag = [&](int rb, int skb) {
    const float* row = sT + (16 * rb + li) * LDA + 32 * skb;
    return to_frag<E>(*reinterpret_cast<const f32x4*>(row + 4 * lg), *reinterpret_cast<const f32x4*>(row + 16 + 4 * lg));
  };

  const float gL = s_gam[63];
  const frag_t<E> id0 = ident_frag<E>(0, li, lg), id1 = ident_frag<E>(1, li, lg);
  const size_t rec_ch = (size_t)ch;

  // K transposes for this wave's feature columns: acc rows s, columns i
  f32x4 kt[4][2];
#pragma unroll
  for (int sb = 0; sb < 4; ++sb) {
    kt[sb][0] = mma(kw[sb], id0, zero4());
    kt[sb][1] = mma(kw[sb], id1, zero4());
  }
  // per-row scales of rows s = 16sb + 4lg + q: beta Gam (W), exp(gL - gamma) (Kt), beta (U)
  auto rowscale = [&](f32x4 x, int sb, int kind) {
    f32x4 y;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int s = 16 * sb + 4 * lg + q;
      const float gs = s_gam[s];
      const float f = kind == 0 ? s_beta[s] * __expf(gs) : (kind == 1 ? __expf(gL - gs) : s_beta[s]);
      y[q] = x[q] * f;
    }
    return y;
  };

  E* Ktf = reinterpret_cast<E*>(p.Ktf);
  E* Wn = reinterpret_cast<E*>(p.Wn);
  E* Ua = reinterpret_cast<E*>(p.Ua);
  constexpr int NJ = D / 16;

  frag_t<E> xw[2][2];
#pragma unroll
  for (int hs = 0; hs < 2; ++hs) {
#pragma unroll
    for (int skb = 0; skb < 2; ++skb) {
      xw[hs][skb] = to_frag<E>(rowscale(kt[2 * skb][hs], 2 * skb, 0), rowscale(kt[2 * skb + 1][hs], 2 * skb + 1, 0));
      const frag_t<E> kk = to_frag<E>(rowscale(kt[2 * skb][hs], 2 * skb, 1), rowscale(kt[2 * skb + 1][hs], 2 * skb + 1, 1));
      const int ib = 2 * w + hs;
      store_rec<E>(Ktf + ((rec_ch * NJ + ib) * 2 + skb) * REC, lane, kk);
    }
  }
  // W^T tiles: acc[i][r] = sum_s Xw[s][i] T[r][s]
#pragma unroll
  for (int rb = 0; rb < 4; ++rb) {
    f32x4 wt0 = zero4(), wt1 = zero4();
#pragma unroll
    for (int skb = 0; skb < 2; ++skb) {
      if (rb <= 1 && skb == 1) continue;
      const frag_t<E> tf = tfrag(rb, skb);
      wt0 = mma(xw[0][skb], tf, wt0);
      wt1 = mma(xw[1][skb], tf, wt1);
    }
    store_rec<E>(Wn + ((rec_ch * 4 + rb) * KB + w) * REC, lane, to_frag<E>(-wt0, -wt1));
  }

  // V transposes and U = T diag(beta) V
#pragma unroll
  for (int hs = 0; hs < 2; ++hs) {
    const frag_t<E> idh = hs ? id1 : id0;
    f32x4 vt[4];
#pragma unroll
    for (int sb = 0; sb < 4; ++sb) vt[sb] = mma(vfw[sb], idh, zero4());
    frag_t<E> xu[2];
#pragma unroll
    for (int skb = 0; skb < 2; ++skb)
      xu[skb] = to_frag<E>(rowscale(vt[2 * skb], 2 * skb, 2), rowscale(vt[2 * skb + 1], 2 * skb + 1, 2));
    const int jb = 2 * w + hs;
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      f32x4 u = zero4();
#pragma unroll
      for (int skb = 0; skb < 2; ++skb) {
        if (rb <= 1 && skb == 1) continue;
        u = mma(tfrag(rb, skb), xu[skb], u);
      }
      store_acc<E>(Ua + ((rec_ch * NJ + jb) * 4 + rb) * AREC, lane, u);
    }
  }
}

// --------------------------------------------------------------------------
// K2: sequential state pass.  One compute wave per (sequence, head, 16-column
// block jb of d_v); the columns of the state are independent, so the compute
// wave needs no communication: its d_k x 16 state stays in accumulator
// registers.  The chunk operands (-W, Kt^T, this block of U, gamma) are
// streamed through an LDS ring by loader waves (ring.h).  A workgroup holds
// CPW column blocks (CPW compute waves sharing the ring's -W and Kt^T).
// Per chunk: store the entering state (fragment-native), V' = U - W h,
// store V', h <- exp(gamma_L) h + Kt^T V'.
template <typename E, int D, int CPW = 1>
struct FwdRing {
  static constexpr int KB = D / 32, NJ = D / 16;
  static constexpr int RECB = REC * (int)sizeof(E);
  static constexpr int oW = 0;
  static constexpr int oK = oW + 4 * KB * RECB;
  static constexpr int oU = oK + NJ * 2 * RECB;
  static constexpr int UB = 4 * AREC * (int)sizeof(E);
  static constexpr int oG = oU + CPW * UB;
  static constexpr int SLOT = oG + 256;
  // at most four waves (one per SIMD, so a compute wave may use 512 VGPRs):
  // with two compute waves, at most two loaders and three slots
  static constexpr int S = CPW == 1 ? ring_slots(SLOT) : (ring_slots(SLOT) < 3 ? ring_slots(SLOT) : 3);
  static constexpr int WAVES = CPW + S - 1;   // compute waves, then loaders
  static constexpr bool FITS = S * SLOT <= 160 * 1024;
  static_assert(WAVES <= 4, "one wave per SIMD");
};

template <typename E, int D, bool ROT, int CPW>
__global__ __launch_bounds__((64 * FwdRing<E, D, CPW>::WAVES)) void k_fwd_state(Params p, int write_ht) {
  using R = FwdRing<E, D, CPW>;
  static_assert(R::FITS, "the ring fits the LDS");
  constexpr int NJ = D / 16, KB = D / 32, S = R::S;
  __shared__ __attribute__((aligned(1024))) char ring[S * R::SLOT];
  const int lane = lane_id(), w = wave_id(), li = lane & 15, lg = lane >> 4;
  const int b = blockIdx.x, xcd = b & 7, slot = b >> 3;
  // CPW column blocks per workgroup (one compute wave each) share its ring:
  // the -W and Kt^T records are read once for all of them
  constexpr int NJP = NJ / CPW;
  const int unit = (slot / NJP) * 8 + xcd, jbp = slot % NJP;
  const int jb0 = CPW * jbp, jb = jb0 + (CPW > 1 && w < CPW ? w : 0);
  if (unit >= p.N * p.H) return;
  const int n = unit / p.H, h = unit - n * p.H;
  const int4 st = seq_info(p, n);
  const int c0 = st.x, nc = st.y;
  // states [N][H][dk][dv]; rows past dk and columns past dv are the padding
  // of D (they start at zero and stay zero)
  const size_t sbase = (size_t)unit * p.kdim * p.vdim;
  const bool col_real = 16 * jb < p.vdim;
  const E* Wn = reinterpret_cast<const E*>(p.Wn);
  const E* Ktf = reinterpret_cast<const E*>(p.Ktf);
  const E* Ua = reinterpret_cast<const E*>(p.Ua);
  E* Hf = reinterpret_cast<E*>(p.Hf);
  E* Vf = reinterpret_cast<E*>(p.Vf);
  // the NJ workgroups of a (sequence, head) read the same -W and Kt^T records;
  // with many of them resident, each starts at its own piece (spread over the
  // L2 channels instead of all on one)
  const int rot = jbp;

  auto issue = [&](int ci) {
    const size_t ch = (size_t)(c0 + ci) * p.H + h;
    char* sl = ring + (ci % S) * R::SLOT;
    if constexpr (ROT) {
      dma_kib_rot(Wn + ch * 4 * KB * REC, sl + R::oW, 4 * KB * R::RECB, lane, rot * (4 * KB * R::RECB / 1024) / NJP);
      dma_kib_rot(Ktf + ch * NJ * 2 * REC, sl + R::oK, NJ * 2 * R::RECB, lane, rot * (NJ * 2 * R::RECB / 1024) / NJP);
    } else {
      dma_kib(Wn + ch * 4 * KB * REC, sl + R::oW, 4 * KB * R::RECB, lane);
      dma_kib(Ktf + ch * NJ * 2 * REC, sl + R::oK, NJ * 2 * R::RECB, lane);
    }
    dma_kib(Ua + (ch * NJ + jb0) * 4 * AREC, sl + R::oU, CPW * R::UB, lane);
    dma_256(p.gamma + ch * 64, sl + R::oG, lane);
  };
  if (w >= CPW && w - CPW < nc) issue(w - CPW);

  if (w < CPW) {
    f32x4 hs[NJ];
#pragma unroll
    for (int ib = 0; ib < NJ; ++ib) {
      if (p.h0 && col_real && 16 * ib < p.kdim) {
        const int ld = p.vdim;
        const float* src = p.h0 + sbase + (size_t)(16 * ib + 4 * lg) * ld + 16 * jb + li;
        hs[ib] = f32x4{src[0], src[ld], src[2 * ld], src[3 * ld]};
      } else {
        hs[ib] = zero4();
      }
    }
    // One chunk's LDS operands.  Where registers allow (bf16, or d = 64),
    // two sets alternate: the next chunk's set is read from its slot while
    // this chunk's second product runs.
    constexpr bool kPipe = sizeof(E) == 2 || D <= 64;
    // Values are kept as read (U in the storage type, raw gamma_L) and
    // converted where the step uses them, so nothing in the step waits for
    // the reads of the next set.
    struct Ops {
      frag_t<E> wf[4][KB], kf[NJ][2];
      quad_t<E> u[4];
      float gL;
    };
    auto read_ops = [&](Ops& o, int ci) {
      const char* sl = ring + (ci % S) * R::SLOT;
#pragma unroll
      for (int rb = 0; rb < 4; ++rb)
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
          o.wf[rb][kb] = load_rec<E>(reinterpret_cast<const E*>(sl + R::oW) + (rb * KB + kb) * REC, lane);
#pragma unroll
      for (int rb = 0; rb < 4; ++rb)
        o.u[rb] = *reinterpret_cast<const quad_t<E>*>(reinterpret_cast<const E*>(sl + R::oU) + (CPW > 1 ? (jb - jb0) * 4 * AREC : 0) + rb * AREC + 4 * lane);
#pragma unroll
      for (int ib = 0; ib < NJ; ++ib)
#pragma unroll
        for (int skb = 0; skb < 2; ++skb)
          o.kf[ib][skb] = load_rec<E>(reinterpret_cast<const E*>(sl + R::oK) + (ib * 2 + skb) * REC, lane);
      o.gL = reinterpret_cast<const float*>(sl + R::oG)[63];
    };
    auto step = [&](int ci, Ops& cur, Ops& nxt) {
      const size_t ch = (size_t)(c0 + ci) * p.H + h;
      frag_t<E> hfr[KB];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) hfr[kb] = to_frag<E>(hs[2 * kb], hs[2 * kb + 1]);
      f32x4 vp[4];
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) vp[rb] = quad_to_f32<E>(cur.u[rb]);
      // V' = U - W h: contraction outermost so consecutive MFMAs are independent
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) vp[rb] = mma(cur.wf[rb][kb], hfr[kb], vp[rb]);
      // decay of the state and V' in the operand type, before the barrier:
      // the empty asm keeps the compiler from sinking them past it onto the
      // second product's critical path
      const float GL = __expf(cur.gL);
#pragma unroll
      for (int ib = 0; ib < NJ; ++ib) {
        hs[ib] = scale4(hs[ib], GL);
        asm volatile("" : "+v"(hs[ib]));
      }
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) store_rec<E>(Hf + ((ch * NJ + jb) * KB + kb) * REC, lane, hfr[kb]);
      frag_t<E> vfr[2];
#pragma unroll
      for (int skb = 0; skb < 2; ++skb) {
        vfr[skb] = to_frag<E>(vp[2 * skb], vp[2 * skb + 1]);
        asm volatile("" : "+v"(vfr[skb]));
      }
      if (kPipe && ci + 1 < nc) {
        // this chunk's reads are complete: release its slot
        wait_lds();
        ring_barrier();
      }
      // fetch the next chunk's operands (the last step reads its own slot
      // again, unused), interleaved with the second product below
      if (kPipe) read_ops(nxt, ci + 1 < nc ? ci + 1 : ci);
      // h <- exp(gamma_L) h + Kt^T V'
#pragma unroll
      for (int skb = 0; skb < 2; ++skb)
#pragma unroll
        for (int ib = 0; ib < NJ; ++ib) hs[ib] = mma(cur.kf[ib][skb], vfr[skb], hs[ib]);
      if (kPipe) {
#pragma unroll
        for (int i = 0; i < 2 * NJ; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);   // LDS reads
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
        }
      }
#pragma unroll
      for (int skb = 0; skb < 2; ++skb) store_rec<E>(Vf + ((ch * NJ + jb) * 2 + skb) * REC, lane, vfr[skb]);
    };
    if constexpr (kPipe) {
      if (nc > 0) {
        Ops A, B;
        ring_barrier();
        read_ops(A, 0);
        for (int ci = 0; ci < nc; ci += 2) {
          step(ci, A, B);
          if (ci + 1 < nc) step(ci + 1, B, A);
        }
      }
    } else {
      Ops A;
      for (int ci = 0; ci < nc; ++ci) {
        ring_barrier();
        read_ops(A, ci);
        step(ci, A, A);
        wait_lds();
      }
    }
    if (write_ht && p.ht && col_real) {
#pragma unroll
      for (int ib = 0; ib < NJ; ++ib) {
        if (16 * ib >= p.kdim) continue;
        const int ld = p.vdim;
        float* dst = p.ht + sbase + (size_t)(16 * ib + 4 * lg) * ld + 16 * jb + li;
        dst[0] = hs[ib][0];
        dst[ld] = hs[ib][1];
        dst[2 * ld] = hs[ib][2];
        dst[3 * ld] = hs[ib][3];
      }
    }
  } else {
    // loader wave w: chunks ci with ci % (S - 1) == w - CPW, S - 1 ahead
    for (int ci = 0; ci < nc; ++ci) {
      const bool mine = (ci % (S - 1)) == w - CPW;
      if (mine) wait_vmem();
      ring_barrier();
      if (mine && ci + S - 1 < nc) issue(ci + S - 1);
    }
  }
}

// --------------------------------------------------------------------------
// K3: output.  Per (chunk, head), D/32 waves.  Q and K are staged in LDS
// once; the masked P = scale (Q K^T) * D is computed one tile per wave in
// turn into LDS; wave w then writes output columns [32w, 32w + 32):
//   O^T[j][r] = Gam_r sum_i h[i][j] Q[r][i] + sum_s V'[s][j] P[r][s]
// reading only its own column blocks of h and V'.
template <typename E, int D>
struct FwdOutSmem {
  static constexpr int TILE = NatTile<E, D>::BYTES;
  static constexpr int LDE = sizeof(E) == 2 ? 72 : 68;
  static constexpr int oQ = 0;
  static constexpr int oK = oQ + TILE;
  static constexpr int oP = oK + TILE;                  // P[r][s], operand type
  static constexpr int oG = oP + 64 * LDE * (int)sizeof(E);
  static constexpr int BYTES = oG + 256;
};

template <typename E, int D, bool NORM>
__global__ __launch_bounds__(64 * (D / 32)) void k_fwd_out(Params p) {
  using S = FwdOutSmem<E, D>;
  constexpr int NJ = D / 16, KB = D / 32, NW = D / 32, LDE = S::LDE;
  __shared__ __attribute__((aligned(16))) char smem[S::BYTES];
  char* tQ = smem + S::oQ;
  char* tK = smem + S::oK;
  E* sP = reinterpret_cast<E*>(smem + S::oP);
  float* s_gam = reinterpret_cast<float*>(smem + S::oG);
  const int ch = blockIdx.x;
  const int H = p.H;
  const int c = ch / H, h = ch - c * H;
  const int4 ct = chunk_info(p, c);
  const int tok0 = ct.x, L = ct.y;
  const int lane = lane_id(), w = wave_id(), li = lane & 15, lg = lane >> 4;
  const int tid = threadIdx.x;
  constexpr int NT = 64 * NW;
  const E* Hf = reinterpret_cast<const E*>(p.Hf);
  const E* Vf = reinterpret_cast<const E*>(p.Vf);
  E* O = reinterpret_cast<E*>(p.o);
  // o: [tokens][H][dv], contiguous
  const size_t rowstride = (size_t)H * p.vdim;
  const size_t base = ((size_t)tok0 * H + h) * p.vdim;

  // every global read is issued before the first use of any of them
  const float gv = p.gamma[(size_t)ch * 64 + lane];
  frag_t<E> hr[2][KB], vr[2][2];   // this wave's column blocks of h and V'
  {
    TileStage<E, D, NT> sq, sk;
    const size_t nb = (size_t)tok0 * H + h;   // reciprocal norms of this chunk's rows, stride H
    // q, k: token stride ldq, dk wide (the output keeps the contiguous layout)
    const size_t xbase = (size_t)tok0 * p.ldq + (size_t)h * p.kdim;
    sq.load(reinterpret_cast<const E*>(p.q) + xbase, (size_t)p.ldq, L, tid, nullptr, 0, p.kdim);
    sk.load(reinterpret_cast<const E*>(p.k) + xbase, (size_t)p.ldq, L, tid, NORM ? p.kinv + nb : nullptr, H, p.kdim);
#pragma unroll
    for (int hs = 0; hs < 2; ++hs) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) hr[hs][kb] = load_rec<E>(Hf + (((size_t)ch * NJ + 2 * w + hs) * KB + kb) * REC, lane);
#pragma unroll
      for (int skb = 0; skb < 2; ++skb) vr[hs][skb] = load_rec<E>(Vf + (((size_t)ch * NJ + 2 * w + hs) * 2 + skb) * REC, lane);
    }
    if (w == 0) s_gam[lane] = gv;
    if constexpr (NORM) sq.norm_rows(L, tid, nullptr, 0);
    sq.store(tQ, tid);
    sk.store(tK, tid);
  }
  // upper blocks of P are zero
  zero_off_blocks<E, true>(sP, LDE, tid, NT);
  __syncthreads();

  // P tiles (r-block rb, s-block sb <= rb), one per wave in turn
  {
    constexpr int TR[10] = {0, 1, 1, 2, 2, 2, 3, 3, 3, 3};
    constexpr int TS[10] = {0, 0, 1, 0, 1, 2, 0, 1, 2, 3};
#pragma unroll
    for (int t = 0; t < 10; ++t) {
      if (t % NW != w) continue;
      const int rb = TR[t], sb = TS[t];
      f32x4 acc = zero4();
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
        acc = mma(tile_frag<E, D>(tK, sb, kb, li, lg), tile_frag<E, D>(tQ, rb, kb, li, lg), acc);
      // lane holds (Q K^T)[r = 16rb + li][s = 16sb + 4lg + q]
      const int r = 16 * rb + li;
      const float gr = s_gam[r];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int s_ = 16 * sb + 4 * lg + q;
        acc[q] = s_ <= r ? p.scale * acc[q] * __expf(gr - s_gam[s_]) : 0.f;
      }
      *reinterpret_cast<quad_t<E>*>(sP + r * LDE + 16 * sb + 4 * lg) = to_quad<E>(acc);
    }
  }
  __syncthreads();

  if (32 * w >= p.vdim) return;   // this wave's output columns are padding of D
#pragma unroll
  for (int rb = 0; rb < 4; ++rb) {
    const int r = 16 * rb + li;
    const float Gr = p.scale * __expf(s_gam[r]);
    frag_t<E> qfr[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) qfr[kb] = tile_frag<E, D>(tQ, rb, kb, li, lg);
    const frag_t<E> pf0 = load_frag_row<E>(sP + r * LDE, lg);
    const frag_t<E> pf1 = load_frag_row<E>(sP + r * LDE + 32, lg);
#pragma unroll
    for (int hs = 0; hs < 2; ++hs) {
      f32x4 acc = zero4();
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) acc = mma(hr[hs][kb], qfr[kb], acc);
      acc = scale4(acc, Gr);
      acc = mma(vr[hs][0], pf0, acc);
      if (rb >= 2) acc = mma(vr[hs][1], pf1, acc);
      if (r < L)
        *reinterpret_cast<quad_t<E>*>(O + base + (size_t)r * rowstride + 32 * w + 16 * hs + 4 * lg) = to_quad<E>(acc);
    }
  }
}

// --------------------------------------------------------------------------
hipError_t launch_plan(const Params& p, hipStream_t s) {
  if (!p.cu) return hipSuccess;  // dense: chunk and sequence info are arithmetic
  Params a = p;
  void* args[] = {&a};
  return hipLaunchKernel((const void*)k_plan, dim3(1), dim3(1024), args, 0, s);
}

template <typename E, int D>
static hipError_t fwd_prep_t(const Params& p, hipStream_t s) {
  if (p.NC == 0) return hipSuccess;
  Params a = p;
  void* args[] = {&a};
  return hipLaunchKernel(p.qk_l2norm ? (const void*)k_fwd_prep<E, D, true> : (const void*)k_fwd_prep<E, D, false>, dim3(p.NC * p.H), dim3(64 * (D / 32)), args, 0, s);
}
template <typename E, int D>
static hipError_t fwd_state_t(const Params& p, bool write_ht, hipStream_t s) {
  if (p.N * p.H == 0) return hipSuccess;
  Params a = p;
  int wh = write_ht ? 1 : 0;
  void* args[] = {&a, &wh};
  // two column blocks per workgroup (a grid past one round; always with rotated
  // reads) where the ring's slots for them fit the LDS
  if constexpr (FwdRing<E, D, 2>::FITS) {
    if (p.state_cpw == 2)
      return hipLaunchKernel((const void*)k_fwd_state<E, D, true, 2>, dim3(state_grid(p.N * p.H, D, 2)),
                             dim3(64 * FwdRing<E, D, 2>::WAVES), args, 0, s);
  }
  return hipLaunchKernel(p.dma_rot ? (const void*)k_fwd_state<E, D, true, 1> : (const void*)k_fwd_state<E, D, false, 1>,
                         dim3(state_grid(p.N * p.H, D)), dim3(64 * FwdRing<E, D, 1>::WAVES), args, 0, s);
}
template <typename E, int D>
static hipError_t fwd_out_t(const Params& p, hipStream_t s) {
  if (p.NC == 0) return hipSuccess;
  Params a = p;
  void* args[] = {&a};
  return hipLaunchKernel(p.qk_l2norm ? (const void*)k_fwd_out<E, D, true> : (const void*)k_fwd_out<E, D, false>, dim3(p.NC * p.H), dim3(64 * (D / 32)), args, 0, s);
}

#define GDN_DISPATCH(fn, ...)                                        \
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

hipError_t launch_fwd_prep(const Params& p, int D, bool is_bf16, hipStream_t s) { GDN_DISPATCH(fwd_prep_t, p, s); }
hipError_t launch_fwd_state(const Params& p, int D, bool is_bf16, bool write_ht, hipStream_t s) {
  GDN_DISPATCH(fwd_state_t, p, write_ht, s);
}
hipError_t launch_fwd_out(const Params& p, int D, bool is_bf16, hipStream_t s) { GDN_DISPATCH(fwd_out_t, p, s); }

}  // namespace gdn
