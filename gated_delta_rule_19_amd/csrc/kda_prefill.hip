// KDA chunked prefill on gfx950: chunk prep (K1), state-carrying chain (K2),
// and the sequence-split planner's prefix scan.
//
// The chunkwise form is the FlashKDA matrix form of "Kimi K3 的架構"
// (hao.cnyes.com), §六 FlashKDA 演算法: per chunk of C = 64 tokens and head,
//   a = exp(cumsum g),  K_decay = Diag(a) K,  Q_decay = Diag(a) Q,
//   K_inv = Diag(a)^-1 K,  K_restore = a[-1] * K_inv,
//   L = StrictTril(Diag(beta) K_decay K_inv^T),  INV = (I + L)^-1,
//   M_qk = tril(Q_decay K_inv^T)   (diagonal kept: an output reads the state
//                                    after its own token's update)
// and then, walking the chunks of a sequence in order,
//   U = INV Diag(beta) (V - K_decay S),  O = Q_decay S + M_qk U,
//   S = Diag(a[-1]) S + K_restore^T U.
//
// Numerics (the decay's lower bound, "Kimi K3.1 Pro 架构完全拆解" §3.2 and
// the orkas.ai page's section on that bound): a chunk-level K_inv would need
// exp(-cumsum g) up to e^320 and overflows fp32.  With g >= -5 every 16-token
// cumulative log-decay lies in (-80, 0], so the products exp(G_r - G_t) needed
// by L and M_qk are factored at 16-token reference points: with p_I the
// cumulative log-decay just before row tile I,
//     exp(G_r - G_t) = exp(G_r - p_I) * exp(p_I - G_t),
// the first factor in (e^-80, 1] for r in tile I, the second <= e^80 on the
// diagonal tile and <= 1 for earlier tiles.  Both fit bf16/fp32, so every
// 16 x 16 tile, the diagonal one included, is one dense MFMA product.
// Q_decay, K_decay and K_restore keep the chunk start/end as reference: their
// factors are <= 1 and underflow only where the exact value is negligible.
//
// INV is computed exactly (up to fp32 rounding) by blocked forward
// substitution over 16 x 16 blocks; any exact method gives the same unique
// inverse of the unit lower-triangular I + L.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

namespace {

constexpr int kThreads = 256;

// Offsets inside one chunk-prep record (element size es).
struct RecOff {
  size_t qd, kd, krt, invb, mqk, ac;
  __host__ __device__ constexpr explicit RecOff(size_t es)
      : qd(0), kd(64 * 128 * es), krt(2 * 64 * 128 * es), invb(3 * 64 * 128 * es),
        mqk(3 * 64 * 128 * es + 64 * 64 * es), ac(3 * 64 * 128 * es + 2 * 64 * 64 * es) {}
};

// The 10 lower (row tile I, column tile J) pairs of a 64 x 64 chunk matrix,
// and the index of each off-diagonal pair among the 6 off-diagonal ones.
__device__ __constant__ int kPairI[10] = {0, 1, 1, 2, 2, 2, 3, 3, 3, 3};
__device__ __constant__ int kPairJ[10] = {0, 0, 1, 0, 1, 2, 0, 1, 2, 3};
__device__ __constant__ int kOffIdx[10] = {-1, 0, -1, 1, 2, -1, 3, 4, 5, -1};
// The 6 off-diagonal pairs (I > J) in the order of kOffIdx, and the 6 upper
// (I < J) tiles.
__device__ __constant__ int kOffI[6] = {1, 2, 2, 3, 3, 3};
__device__ __constant__ int kOffJ[6] = {0, 0, 1, 0, 1, 2};
__device__ __constant__ int kUpI[6] = {0, 0, 0, 1, 1, 2};
__device__ __constant__ int kUpJ[6] = {1, 2, 3, 2, 3, 3};

template <typename T> constexpr int pad_elems() { return 16 / (int)sizeof(T) * 2; }

// Workgroup barrier that orders LDS only: outstanding global loads stay in
// flight across it (a full __syncthreads() would wait for them too).
__device__ __forceinline__ void lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

} // namespace

// ---------------------------------------------------------------------------
// K1: chunk prep.  One workgroup per (chunk, head), chunk-parallel.  With
// has_q == 0 (segment transitions need no outputs) q is not a real input:
// Q_decay and M_qk are then 0.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(kThreads) void k1_kernel(const ChunkDesc *__restrict__ chunks,
                                                      int32_t H, const T *__restrict__ q,
                                                      const T *__restrict__ k,
                                                      const T *__restrict__ g,
                                                      const T *__restrict__ beta,
                                                      uint8_t *__restrict__ ws, int has_q) {
  constexpr int P = pad_elems<T>();
  constexpr int LD = kD + P;                 // operand row stride (elements)
  constexpr size_t OPB = (size_t)kC * LD * sizeof(T);
  constexpr RecOff off(sizeof(T));
  // Operand region: Q_loc, K_loc, K_start, K_end (4 x [C][LD] of T).  After
  // the MFMA phase it is reused for L, INV and a scratch block (fp32).
  __shared__ __attribute__((aligned(16))) uint8_t smem[4 * OPB];
  __shared__ float sP[5][kD];   // reference log-decays p_0..p_3 and G_last
  __shared__ float sF[6][kD];   // exp(p_I - p_{J+1}) for off-diagonal pairs
  __shared__ float sBeta[kC];
  __shared__ float sTot[kD];

  T(*sQl)[LD] = reinterpret_cast<T(*)[LD]>(smem);
  T(*sKl)[LD] = reinterpret_cast<T(*)[LD]>(smem + OPB);
  T(*sKs)[LD] = reinterpret_cast<T(*)[LD]>(smem + 2 * OPB);
  T(*sKe)[LD] = reinterpret_cast<T(*)[LD]>(smem + 3 * OPB);
  constexpr int LF = kC + 1;
  float(*sL)[LF] = reinterpret_cast<float(*)[LF]>(smem);
  float(*sInv)[LF] = reinterpret_cast<float(*)[LF]>(smem + kC * LF * 4);
  float(*sTmp)[LF] = reinterpret_cast<float(*)[LF]>(smem + 2 * kC * LF * 4);
  static_assert((2 * kC + 16) * LF * 4 <= 4 * OPB, "aliasing fits");

  const int ci = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  const ChunkDesc cd = chunks[ci];
  const int len = cd.len;
  const int c = tid & (kD - 1);
  const int half = tid >> 7;
  const int64_t rowstride = (int64_t)H * kD;
  uint8_t *rec = ws + ((int64_t)ci * H + h) * k1_record_bytes(sizeof(T));
  T *Qd = reinterpret_cast<T *>(rec + off.qd);
  T *Kd = reinterpret_cast<T *>(rec + off.kd);
  T *KrT = reinterpret_cast<T *>(rec + off.krt);
  T *INVb = reinterpret_cast<T *>(rec + off.invb);
  T *Mqk = reinterpret_cast<T *>(rec + off.mqk);
  float *ac = reinterpret_cast<float *>(rec + off.ac);

  // ---- loads: every row index is clamped into the chunk, so all loads are
  // unconditional and in flight together; padded rows are zeroed afterwards.
  T graw[32], qraw[32], kraw[32];
  {
    const int64_t base = cd.tok0 * rowstride + (int64_t)h * kD + c;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const int rr = min(half * 32 + i, len - 1);
      const int64_t off = base + (int64_t)rr * rowstride;
      graw[i] = g[off];
      kraw[i] = k[off];
      qraw[i] = q[off];
    }
  }
  const float bval = to_f32(beta[(cd.tok0 + min(tid & (kC - 1), len - 1)) * H + h]);
  if (tid < kC)
    sBeta[tid] = (tid < len) ? bval : 0.f;

  // ---- phase 1: inclusive cumulative log-decay per channel -------------
  float G[32];
  {
    float run = 0.f;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const float gv = (half * 32 + i < len) ? to_f32(graw[i]) : 0.f;
      run += gv;
      G[i] = run;
    }
    if (half == 0)
      sTot[c] = run;
  }
  lds_sync();
  if (half == 1) {
    const float base = sTot[c];
#pragma unroll
    for (int i = 0; i < 32; ++i)
      G[i] += base;
    sP[3][c] = G[15];
    sP[4][c] = G[31];
  } else {
    sP[0][c] = 0.f;
    sP[1][c] = G[15];
    sP[2][c] = G[31];
  }
  lds_sync();

  // ---- phase 2: decayed operands ----------------------------------------
  {
    const float pC = sP[4][c];
    float krv[32];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const int I = half * 2 + tt;
      const float pI = sP[I][c], pI1 = sP[I + 1][c];
      const float eP = __expf(pI);         // exp(p_I)           <= 1
      const float eR = __expf(pC - pI1);   // exp(G_last - p_I+1) <= 1
#pragma unroll
      for (int ii = 0; ii < 16; ++ii) {
        const int i = tt * 16 + ii;
        const int r = half * 32 + i;
        const bool ok = r < len;
        const float qv = (ok && has_q) ? to_f32(qraw[i]) : 0.f;
        const float kv = ok ? to_f32(kraw[i]) : 0.f;
        const float eloc = __expf(G[i] - pI);  // (e^-80, 1]
        const float est = __expf(pI - G[i]);   // [1, e^80)
        const float eend = __expf(pI1 - G[i]); // (e^-80, 1]
        sQl[r][c] = from_f32<T>(qv * eloc);
        sKl[r][c] = from_f32<T>(kv * eloc);
        sKs[r][c] = from_f32<T>(kv * est);
        sKe[r][c] = from_f32<T>(kv * eend);
        const float ga = eloc * eP;            // exp(G_r)
        Qd[r * kD + c] = from_f32<T>(qv * ga);
        Kd[r * kD + c] = from_f32<T>(kv * ga);
        krv[i] = kv * (eend * eR);             // exp(G_last - G_r) k
      }
    }
    // K_restore^T row c, tokens half*32 .. +31 (contiguous)
    T *kr = KrT + c * kC + half * 32;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float x[8];
#pragma unroll
      for (int e = 0; e < 8; ++e)
        x[e] = krv[8 * j + e];
      store8(kr + 8 * j, x);
    }
    if (half == 0)
      ac[c] = __expf(pC);
    // off-diagonal factors exp(p_I - p_{J+1}), I > J: 6 pairs x 128 channels
    for (int p = half; p < 6; p += 2)
      sF[p][c] = __expf(sP[kOffI[p]][c] - sP[kOffJ[p] + 1][c]);
  }
  lds_sync();

  // ---- phase 3: L and M_qk tiles on MFMA ---------------------------------
  const int wv = tid >> 6, lane = tid & 63, lr = lane & 15, lg = lane >> 4;
  f32x4 accL[3], accM[3];
#pragma unroll
  for (int pp = 0; pp < 3; ++pp) {
    accL[pp] = f32x4{0.f, 0.f, 0.f, 0.f};
    accM[pp] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int p = wv + 4 * pp;
    if (p < 10) {
      const int I = kPairI[p], J = kPairJ[p];
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int kb = 32 * s + 8 * lg;
        const Frag<T> aK = load_frag(&sKl[16 * I + lr][kb]);
        const Frag<T> aQ = load_frag(&sQl[16 * I + lr][kb]);
        Frag<T> b;
        if (I == J) {
          b = load_frag(&sKs[16 * J + lr][kb]);
        } else {
          const Frag<T> e = load_frag(&sKe[16 * J + lr][kb]);
          float x[8];
          frag_to_f32(e, x);
          const float *f = &sF[kOffIdx[p]][kb];
#pragma unroll
          for (int j = 0; j < 8; ++j)
            x[j] *= f[j];
          b = frag_from_f32<T>(x);
        }
        mma(accL[pp], aK, b);
        mma(accM[pp], aQ, b);
      }
    }
  }
  lds_sync(); // operand region is now free for L / INV

  // L (beta-scaled rows, strictly lower) to LDS; M_qk (lower incl. diagonal)
  // straight to the record.
#pragma unroll
  for (int pp = 0; pp < 3; ++pp) {
    const int p = wv + 4 * pp;
    if (p < 10) {
      const int I = kPairI[p], J = kPairJ[p];
      const int col = 16 * J + lr;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 16 * I + 4 * lg + i;
        sL[row][col] = (col < row) ? sBeta[row] * accL[pp][i] : 0.f;
        Mqk[row * kC + col] = from_f32<T>((col <= row) ? accM[pp][i] : 0.f);
      }
    }
  }
  // zero the upper tiles (J > I) of L, INV and M_qk
  for (int e = tid; e < 6 * 256; e += kThreads) {
    const int t = e >> 8, r = (e >> 4) & 15, cc = e & 15;
    const int row = 16 * kUpI[t] + r, col = 16 * kUpJ[t] + cc;
    sL[row][col] = 0.f;
    sInv[row][col] = 0.f;
    Mqk[row * kC + col] = from_f32<T>(0.f);
  }
  lds_sync();

  // ---- phase 4: INV = (I + L)^-1 by blocked forward substitution ---------
  if (tid < 64) {
    // diagonal block b, column j:  x = (I + L_bb)^-1 e_j
    const int b = tid >> 4, j = tid & 15;
    float x[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float acc = (i == j) ? 1.f : 0.f;
#pragma unroll
      for (int m = 0; m < i; ++m)
        acc -= sL[16 * b + i][16 * b + m] * x[m];
      x[i] = acc;
    }
#pragma unroll
    for (int i = 0; i < 16; ++i)
      sInv[16 * b + i][16 * b + j] = x[i];
  }
  lds_sync();
  for (int bi = 1; bi < 4; ++bi) {
    // T_j = sum_{m=j}^{bi-1} L[bi][m] INV[m][j]   for j < bi
    for (int e = tid; e < bi * 256; e += kThreads) {
      const int j = e >> 8, r = (e >> 4) & 15, cc = e & 15;
      float acc = 0.f;
      for (int m = j; m < bi; ++m)
#pragma unroll
        for (int u = 0; u < 16; ++u)
          acc += sL[16 * bi + r][16 * m + u] * sInv[16 * m + u][16 * j + cc];
      sTmp[r][16 * j + cc] = acc;
    }
    lds_sync();
    // INV[bi][j] = -INV[bi][bi] T_j
    for (int e = tid; e < bi * 256; e += kThreads) {
      const int j = e >> 8, r = (e >> 4) & 15, cc = e & 15;
      float acc = 0.f;
#pragma unroll
      for (int u = 0; u < 16; ++u)
        acc += sInv[16 * bi + r][16 * bi + u] * sTmp[u][16 * j + cc];
      sInv[16 * bi + r][16 * j + cc] = -acc;
    }
    lds_sync();
  }

  // INV * Diag(beta) to the record, 16 contiguous elements per thread
  {
    const int row = tid >> 2, c0 = (tid & 3) * 16;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      float x[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int col = c0 + 8 * j + e;
        x[e] = sInv[row][col] * sBeta[col];
      }
      store8(INVb + row * kC + c0 + 8 * j, x);
    }
  }
}

// ---------------------------------------------------------------------------
// K2: state-carrying chain.  One workgroup per (chain, head, column block of
// kBV state columns).  The columns of V, U, O and S are independent, so a
// head's state splits across column blocks with no exchange.
//   MODE 0: prefill / replay, width dv; writes o and the exit state.
//   MODE 1: segment pass, width dk + dv of [S~ | M] from [0 | I] with values
//           [V | 0]; the exit state's S~ part goes to out_a, M part to out_b.
// The loop is latency-bound (S -> W -> U -> S per chunk), so every global
// operand of chunk i+1 is loaded into registers while chunk i is computed,
// and the workgroup barriers order LDS only.
// ---------------------------------------------------------------------------
template <typename T, int NCT> struct ChunkOps {
  Frag<T> kd[4], qd[4], invb[2], mqk[2], krt[2][2];
  f32x4 ac[2];
  T v[NCT][4];
};

template <typename T, int MODE, int NCT>
__device__ __forceinline__ void load_chunk_ops(ChunkOps<T, NCT> &op, const uint8_t *rec,
                                               const T *vbase, int len, int64_t rowstride,
                                               int wv, int lr, int lg) {
  constexpr RecOff off(sizeof(T));
  const T *Qd = reinterpret_cast<const T *>(rec + off.qd);
  const T *Kd = reinterpret_cast<const T *>(rec + off.kd);
  const T *KrT = reinterpret_cast<const T *>(rec + off.krt);
  const T *INVb = reinterpret_cast<const T *>(rec + off.invb);
  const T *Mqk = reinterpret_cast<const T *>(rec + off.mqk);
  const float *ac = reinterpret_cast<const float *>(rec + off.ac);
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    op.kd[s] = load_frag(Kd + (16 * wv + lr) * kD + 32 * s + 8 * lg);
    if (MODE == 0)
      op.qd[s] = load_frag(Qd + (16 * wv + lr) * kD + 32 * s + 8 * lg);
  }
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    op.invb[s] = load_frag(INVb + (16 * wv + lr) * kC + 32 * s + 8 * lg);
    if (MODE == 0)
      op.mqk[s] = load_frag(Mqk + (16 * wv + lr) * kC + 32 * s + 8 * lg);
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
      op.krt[rt][s] = load_frag(KrT + (16 * (2 * wv + rt) + lr) * kC + 32 * s + 8 * lg);
  }
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
    op.ac[rt] = *reinterpret_cast<const f32x4 *>(ac + 16 * (2 * wv + rt) + 4 * lg);
  // V rows clamped into the chunk (rows past its end are zeroed at use)
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int rr = min(16 * wv + 4 * lg + i, len - 1);
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
      op.v[ct][i] = vbase[(int64_t)rr * rowstride + 16 * ct + lr];
  }
}

template <typename T, int MODE>
__global__ __launch_bounds__(kThreads) void k2_kernel(
    const ChainDesc *__restrict__ chains, int32_t H, const uint8_t *__restrict__ ws,
    const T *__restrict__ v, T *__restrict__ o, const float *__restrict__ init,
    const float *__restrict__ sin, float *__restrict__ out_a, float *__restrict__ out_b) {
  constexpr int P = pad_elems<T>();
  constexpr int LDS_S = kD + P; // Sb row stride: [col][channel]
  constexpr int LDS_C = kC + P; // VWb / Ub row stride: [col][token]
  constexpr int NCT = kBV / 16;
  constexpr size_t RB = k1_record_bytes(sizeof(T));
  __shared__ __attribute__((aligned(16))) T Sb[kBV][LDS_S];
  __shared__ __attribute__((aligned(16))) T VWb[kBV][LDS_C];
  __shared__ __attribute__((aligned(16))) T Ub[kBV][LDS_C];

  const ChainDesc cd = chains[blockIdx.x];
  const int h = blockIdx.y;
  const int col0 = blockIdx.z * kBV;
  const bool mpart = (MODE == 1) && (col0 >= kD);
  const int vcol0 = mpart ? col0 - kD : col0;
  const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63, lr = lane & 15, lg = lane >> 4;
  const int64_t rowstride = (int64_t)H * kD;
  const int nch = (cd.ntok + kC - 1) / kC;

  // state rows 16*(2wv+rt) + 4lg + i, columns vcol0 + 16ct + lr
  f32x4 sacc[2][NCT];
  {
    const float *ip = nullptr;
    if (MODE == 0) {
      if (cd.init_idx >= 0)
        ip = init + ((int64_t)cd.init_idx * H + h) * (kD * kD);
      else if (cd.init_idx <= -2)
        ip = sin + ((int64_t)(-2 - cd.init_idx) * H + h) * (kD * kD);
    }
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = 16 * (2 * wv + rt) + 4 * lg + i;
          const int col = vcol0 + 16 * ct + lr;
          sacc[rt][ct][i] = ip ? ip[row * kD + col] : ((mpart && row == col) ? 1.f : 0.f);
        }
  }

  if (nch > 0) {
    const T *vchain = v + cd.tok0 * rowstride + (int64_t)h * kD + vcol0;
    const uint8_t *rec0 = ws + ((int64_t)cd.chunk0 * H + h) * RB;
    ChunkOps<T, NCT> cur, nxt;
    load_chunk_ops<T, MODE, NCT>(cur, rec0, vchain, min(kC, cd.ntok), rowstride, wv, lr, lg);

    for (int ch = 0; ch < nch; ++ch) {
      const int len = min(kC, cd.ntok - ch * kC);
      const int64_t tok = cd.tok0 + (int64_t)ch * kC;
      {
        // prefetch chunk ch+1 (the last chunk reloads itself; harmless)
        const int cn = min(ch + 1, nch - 1);
        load_chunk_ops<T, MODE, NCT>(nxt, rec0 + (int64_t)cn * H * RB,
                                     vchain + (int64_t)cn * kC * rowstride,
                                     min(kC, cd.ntok - cn * kC), rowstride, wv, lr, lg);
      }

      // (1) S -> Sb (MFMA B operand, K = channel)
#pragma unroll
      for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
          store4(&Sb[16 * ct + lr][16 * (2 * wv + rt) + 4 * lg], sacc[rt][ct][0],
                 sacc[rt][ct][1], sacc[rt][ct][2], sacc[rt][ct][3]);
      lds_sync();

      // (2) W = K_decay S and (mode 0) O = Q_decay S for token tile wv
      f32x4 W[NCT], Oa[NCT];
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        W[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
        Oa[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int kb = 32 * s + 8 * lg;
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
          const Frag<T> b = load_frag(&Sb[16 * ct + lr][kb]);
          mma(W[ct], cur.kd[s], b);
          if (MODE == 0)
            mma(Oa[ct], cur.qd[s], b);
        }
      }

      // (3) V - W -> VWb (B operand, K = token)
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        float x[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = 16 * wv + 4 * lg + i;
          const float vv = (!mpart && row < len) ? to_f32(cur.v[ct][i]) : 0.f;
          x[i] = vv - W[ct][i];
        }
        store4(&VWb[16 * ct + lr][16 * wv + 4 * lg], x[0], x[1], x[2], x[3]);
      }
      lds_sync();

      // (4) U = INV Diag(beta) (V - W)
      f32x4 U[NCT];
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
        U[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const int kb = 32 * s + 8 * lg;
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
          const Frag<T> b = load_frag(&VWb[16 * ct + lr][kb]);
          mma(U[ct], cur.invb[s], b);
        }
      }
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
        store4(&Ub[16 * ct + lr][16 * wv + 4 * lg], U[ct][0], U[ct][1], U[ct][2], U[ct][3]);
      lds_sync();

      // (5) O = Q_decay S + M_qk U
      if (MODE == 0) {
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const int kb = 32 * s + 8 * lg;
#pragma unroll
          for (int ct = 0; ct < NCT; ++ct) {
            const Frag<T> b = load_frag(&Ub[16 * ct + lr][kb]);
            mma(Oa[ct], cur.mqk[s], b);
          }
        }
        T *orow = o + tok * rowstride + (int64_t)h * kD + vcol0;
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int row = 16 * wv + 4 * lg + i;
            if (row < len)
              orow[(int64_t)row * rowstride + 16 * ct + lr] = from_f32<T>(Oa[ct][i]);
          }
      }

      // (6) S = Diag(a_last) S + K_restore^T U
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) {
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
          sacc[rt][ct] *= cur.ac[rt];
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const int kb = 32 * s + 8 * lg;
#pragma unroll
          for (int ct = 0; ct < NCT; ++ct) {
            const Frag<T> b = load_frag(&Ub[16 * ct + lr][kb]);
            mma(sacc[rt][ct], cur.krt[rt][s], b);
          }
        }
      }
      cur = nxt;
    }
  }

  float *fp = nullptr;
  if (cd.final_idx >= 0) {
    float *base = (MODE == 1 && mpart) ? out_b : out_a;
    fp = base + ((int64_t)cd.final_idx * H + h) * (kD * kD);
  }
  if (fp) {
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = 16 * (2 * wv + rt) + 4 * lg + i;
          fp[row * kD + vcol0 + 16 * ct + lr] = sacc[rt][ct][i];
        }
  }
}

// ---------------------------------------------------------------------------
// Planner scan: entry states of the segments of one split sequence,
//   Sin[0] = S_0,   Sin[j+1] = S~_j + M_j Sin[j]
// ("部署 Kimi K3：从 KDA Kernel 到 Fleet 调度", §二: S = S~ + M S_in, pairs
// compose associatively).  Serial over segments, parallel over heads and
// column blocks of kScanBV state columns.  fp32 throughout.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void scan_kernel(const ScanDesc *__restrict__ descs,
                                                        int32_t H,
                                                        const float *__restrict__ Mseg,
                                                        const float *__restrict__ Stseg,
                                                        const float *__restrict__ init,
                                                        float *__restrict__ sin) {
  static_assert(kScanBV == 8, "thread map assumes 8 columns");
  __shared__ __attribute__((aligned(16))) float sS[kD][kScanBV];
  const ScanDesc d = descs[blockIdx.x];
  const int h = blockIdx.y;
  const int col0 = blockIdx.z * kScanBV;
  const int tid = threadIdx.x;
  const int r = tid >> 1, cq = (tid & 1) * 4;
  const int64_t mat = (int64_t)kD * kD;

  f32x4 cur = {0.f, 0.f, 0.f, 0.f};
  if (d.init_idx >= 0)
    cur = *reinterpret_cast<const f32x4 *>(init + ((int64_t)d.init_idx * H + h) * mat +
                                           r * kD + col0 + cq);
  *reinterpret_cast<f32x4 *>(sin + ((int64_t)d.sin0 * H + h) * mat + r * kD + col0 + cq) = cur;
  *reinterpret_cast<f32x4 *>(&sS[r][cq]) = cur;
  __syncthreads();

  for (int j = 0; j + 1 < d.nseg; ++j) {
    const float *Mj = Mseg + ((int64_t)(d.pair0 + j) * H + h) * mat + r * kD;
    const float *Sj = Stseg + ((int64_t)(d.pair0 + j) * H + h) * mat + r * kD;
    f32x4 acc = *reinterpret_cast<const f32x4 *>(Sj + col0 + cq);
#pragma unroll 4
    for (int m = 0; m < kD; m += 4) {
      const f32x4 mr = *reinterpret_cast<const f32x4 *>(Mj + m);
#pragma unroll
      for (int mm = 0; mm < 4; ++mm)
        acc += mr[mm] * *reinterpret_cast<const f32x4 *>(&sS[m + mm][cq]);
    }
    __syncthreads();
    *reinterpret_cast<f32x4 *>(&sS[r][cq]) = acc;
    *reinterpret_cast<f32x4 *>(sin + ((int64_t)(d.sin0 + j + 1) * H + h) * mat + r * kD +
                               col0 + cq) = acc;
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
hipError_t launch_k1(int elt, const ChunkDesc *chunks, int32_t nchunks, int32_t H,
                     const void *q, const void *k, const void *g, const void *beta, void *ws,
                     hipStream_t s) {
  if (nchunks == 0)
    return hipSuccess;
  dim3 grid((unsigned)nchunks, (unsigned)H), block(kThreads);
  // without q, k stands in as a readable buffer of the same shape
  const int has_q = q != nullptr;
  const void *qq = has_q ? q : k;
  if (elt == 1)
    k1_kernel<bf16><<<grid, block, 0, s>>>(chunks, H, (const bf16 *)qq, (const bf16 *)k,
                                           (const bf16 *)g, (const bf16 *)beta,
                                           (uint8_t *)ws, has_q);
  else
    k1_kernel<float><<<grid, block, 0, s>>>(chunks, H, (const float *)qq, (const float *)k,
                                            (const float *)g, (const float *)beta,
                                            (uint8_t *)ws, has_q);
  return hipGetLastError();
}

hipError_t launch_k2(int elt, int mode, const ChainDesc *chains, int32_t nchains, int32_t H,
                     const void *ws, const void *v, void *o, const float *init,
                     const float *sin, float *final_a, float *final_b, hipStream_t s) {
  if (nchains == 0)
    return hipSuccess;
  const unsigned width = mode == 1 ? 2 * kD : kD;
  dim3 grid((unsigned)nchains, (unsigned)H, width / kBV), block(kThreads);
  const uint8_t *w = (const uint8_t *)ws;
  if (elt == 1) {
    if (mode == 1)
      k2_kernel<bf16, 1><<<grid, block, 0, s>>>(chains, H, w, (const bf16 *)v,
                                                (bf16 *)o, init, sin, final_a, final_b);
    else
      k2_kernel<bf16, 0><<<grid, block, 0, s>>>(chains, H, w, (const bf16 *)v,
                                                (bf16 *)o, init, sin, final_a, final_b);
  } else {
    if (mode == 1)
      k2_kernel<float, 1><<<grid, block, 0, s>>>(chains, H, w, (const float *)v,
                                                 (float *)o, init, sin, final_a, final_b);
    else
      k2_kernel<float, 0><<<grid, block, 0, s>>>(chains, H, w, (const float *)v,
                                                 (float *)o, init, sin, final_a, final_b);
  }
  return hipGetLastError();
}

hipError_t launch_scan(const ScanDesc *descs, int32_t ndesc, int32_t H, const float *Mseg,
                       const float *Stseg, const float *init, float *sin, hipStream_t s) {
  if (ndesc == 0)
    return hipSuccess;
  dim3 grid((unsigned)ndesc, (unsigned)H, kD / kScanBV), block(kThreads);
  scan_kernel<<<grid, block, 0, s>>>(descs, H, Mseg, Stseg, init, sin);
  return hipGetLastError();
}

} // namespace kda
