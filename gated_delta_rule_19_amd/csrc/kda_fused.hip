// KDA chunked prefill with chunk prep and state carry fused in one kernel
// (bf16 inputs, fp32 state and accumulation).
//
// The mathematics is the two-kernel path's (kda_prefill.hip): the FlashKDA
// chunk form of "Kimi K3 的架構" (hao.cnyes.com) §六, with the 16-token
// reference points that the decay's lower bound allows ("Kimi K3.1 Pro
// 架构完全拆解" §3.2).  What changes is where the chunk-prep results live:
// here they never leave the compute unit, so the only HBM traffic is the
// layer's own inputs and outputs (q, k, v, g, beta in; o and states out).
//
// One workgroup of 8 waves owns one (chain, head, column block of 64 NCT
// state columns).  The waves have two roles that run side by side, two waves
// per SIMD:
//   waves 0-3, state: wave w carries columns 16 NCT w .. 16 NCT w + 16 NCT - 1
//     of the column block through the chunks, S in MFMA accumulators:
//       W = K_decay S,  O = Q_decay S,  U = INV Diag(beta) (V - W),
//       O += M_qk U,  S = Diag(a_last) S + K_restore^T U;
//   waves 4-7, prep: wave p owns token tile p (16 tokens) of chunk c and
//     builds its part of that chunk's record: cumulative log-decay, decayed
//     q / k, K_restore, L and M_qk on MFMA, INV = (I + L)^-1.
// A chunk step is four stages separated by workgroup barriers.  Every record
// region is rewritten by the prep only in a stage after the one in which the
// state waves read it, so one record buffer serves both roles:
//   stage | state waves                            | prep waves (chunk c)
//   A     | -                                      | tile scan, Q_loc/K_loc/K_start, diagonal L, M_qk tiles
//   B     | U, O += M_qk U, store o, S update      | factors, K_decay/Q_decay -> record, off-diagonal tiles
//         |   (chunk c - 1)                        |
//   C     | -                                      | L, M_qk, K_restore^T, a_last -> record; diagonal INV blocks
//   D     | W = K_decay S, O = Q_decay S (chunk c) | off-diagonal blocks of INV -> record
//
// Prep lane layout: prep wave p, lane (lr, lg) = (lane % 16, lane / 16) holds
// token 16 p + lr and, for k-step s = 0..3, channels 32 s + 8 lg .. + 7: one
// 16-byte load per input and k-step, the MFMA A-fragment layout of the L /
// M_qk products, and one 16-byte row piece of Q_decay / K_decay.  The tile's
// cumulative sum of g runs across the 16 lanes of a DPP row.
//
// State row order: the state waves keep channel kperm(p) in accumulator row
// p (p = 16 ct + 4 lg + i).  Packing two stacked accumulator tiles then gives
// exactly channels 32 s + 8 lg .. + 7 in lane (., lg), the B operand of the
// K = channels products, so the state feeds W and O without moving data
// between lanes.  K_restore^T and a_last are stored in the same row order.
//
// Numerics, with G the inclusive cumulative log-decay from the chunk start,
// p_I = G before token tile I, G_loc = G - p_I and G_C the chunk total:
//   Q_loc = q e^{G_loc},  K_loc = k e^{G_loc}            (<= |q|, |k|)
//   K_st  = k e^{-G_loc}                                 (<= e^80 |k|)
//   L_IJ  = K_loc,I (K_st,J e^{p_I - p_J})^T  for J < I;  K_loc,I K_st,I^T on the diagonal
//   Q_decay = q e^{G_loc + p_I},  K_decay = k e^{G_loc + p_I},  K_restore = k e^{G_C - p_I - G_loc}
// Every exponent is <= 0 except K_st's (< 80); a factor that underflows does
// so only where the exact product is below e^-20 of its neighbours.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

namespace {

constexpr int kFWaves = 8;
constexpr int kFThreads = 64 * kFWaves;
constexpr int kLdD = kD + 8; // bf16 rows of 128 (272 B: 16 rows of a fragment read hit distinct banks)
constexpr int kLdC = kC + 8; // bf16 rows of 64 (144 B)
constexpr int kLdL = kC + 4; // fp32 rows of 64
constexpr int kLdB = 20;     // fp32 16 x 16 blocks
constexpr float kLog2e = 1.4426950408889634f;

// The 6 off-diagonal tile pairs (I, J), I > J, and the prep wave that
// computes each (two waves take two pairs, two take one).  A pair's A
// operand (K_loc / Q_loc rows of tile I) is in registers when the wave owns
// tile I, else it comes from the copy tile 3 leaves in LDS.
//   wave 0: (3,0)   wave 1: (1,0) (3,1)   wave 2: (2,0) (2,1)   wave 3: (3,2)
__host__ __device__ constexpr int pair_count(int w) { return (w == 1 || w == 2) ? 2 : 1; }
__host__ __device__ constexpr int pair_I(int w, int n) {
  return w == 0 ? 3 : (w == 1 ? (n == 0 ? 1 : 3) : (w == 2 ? 2 : 3));
}
__host__ __device__ constexpr int pair_J(int w, int n) {
  return w == 0 ? 0 : (w == 1 ? (n == 0 ? 0 : 1) : (w == 2 ? (n == 0 ? 0 : 1) : 2));
}

template <int NCT> struct FusedSmem {
  // the chunk record (state waves read it, prep waves rewrite it)
  bf16 Qd[kC][kLdD];   // Q_decay, rows = tokens, columns = channels
  bf16 Kd[kC][kLdD];   // K_decay
  bf16 KrT[kD][kLdC];  // K_restore^T, row p = channel kperm(p), columns kperm(token)
  bf16 INVb[kC][kLdC]; // INV Diag(beta), columns kperm(token)
  bf16 Mqk[kC][kLdC];  // M_qk, columns kperm(token)
  float aL[kD];        // a_last, entry p = channel kperm(p)
  // v of each state wave's columns: 64 rows x 16 NCT columns
  bf16 sv[4][kC * 16 * NCT];
  // prep scratch
  float Tot[4][kD]; // per-tile totals of g
  union {
    struct {
      bf16 Kst[4][16][kLdD]; // K_start per tile (stage A -> B)
      bf16 Aq3[2][16][kLdD]; // K_loc, Q_loc of tile 3 (stage A -> B)
    } ab;
    float Pow[4][2][16][kLdB]; // per prep wave: N^2, N^4 of its diagonal block (stage C)
  } x;
  float L[kC][kLdL];       // L = StrictTril(Diag(beta) K_decay K_inv^T), fp32
  float Dinv[4][16][kLdB]; // inverted diagonal blocks of I + L
  float Beta[kC];
  float Iq[kC], Ik[kC];    // prologue: 1 / |q|, 1 / |k| per token (stage A -> B)
  float Red[4][kC];        // output norm: per state wave, partial sums of o^2 per token
  float Scl[4][kC];        // output norm: each state wave's copy of the row scales
  float Fac[4][2][kD];     // per tile, log2 units: p_I, G_C - p_I
  float Foff[6][kD];       // e^{p_I - p_J} for the off-diagonal pairs
};

// index of the tile pair (I, J), I > J, among the 6 off-diagonal pairs
__device__ __forceinline__ int off_pair(int I, int J) { return I * (I - 1) / 2 + J; }



} // namespace

// PRO: the prologue (gate logits -> log decay, q / k L2 norm) is compiled in;
// which of its steps run is decided by A_log != null and qk_eps > 0.
// EPI: o leaves through the output norm and gate.
template <int NCT, bool PRO, bool EPI>
__global__ __launch_bounds__(kFThreads) void fused_kernel(
    const ChainDesc *__restrict__ chains, int32_t H, const bf16 *__restrict__ q,
    const bf16 *__restrict__ k, const bf16 *__restrict__ v, const bf16 *__restrict__ g,
    const bf16 *__restrict__ beta, bf16 *__restrict__ o, const float *__restrict__ init,
    const float *__restrict__ sin, float *__restrict__ final_state, float *__restrict__ ckpt,
    const float *__restrict__ A_log, float g_min, float qk_eps, const bf16 *__restrict__ ogate,
    const float *__restrict__ onw, float oeps) {
  using Sm = FusedSmem<NCT>;
  __shared__ __attribute__((aligned(16))) Sm sm;
  constexpr int VW = 16 * NCT; // state columns per state wave

  const ChainDesc cd = chains[blockIdx.x];
  const int h = blockIdx.y;
  const int col0 = blockIdx.z * (4 * VW);
  const int tid = threadIdx.x;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t rowstride = (int64_t)H * kD;
  const int nch = (cd.ntok + kC - 1) / kC;

  // The upper 16 x 16 tiles of M_qk and INV Diag(beta) are zero and are
  // never written again.
  for (int e = tid; e < 6 * 256; e += kFThreads) {
    const int t = e >> 8, r = (e >> 4) & 15, c = e & 15;
    const int bi = t < 3 ? 0 : (t < 5 ? 1 : 2);
    const int bj = t < 3 ? t + 1 : (t < 5 ? t - 1 : 3);
    sm.INVb[16 * bi + r][kperm(16 * bj + c)] = static_cast<bf16>(0.f);
    sm.Mqk[16 * bi + r][kperm(16 * bj + c)] = static_cast<bf16>(0.f);
  }
  lds_barrier();

  if (wv < 4) {
    // =========================== state waves ===========================
    const int lane = tid & 63, lr = lane & 15, lg = lane >> 4;
    const int wcol = col0 + VW * wv + lr; // this lane's column in tile c: wcol + 16 c
    f32x4 S[NCT][8];                      // rows p = 16 ct + 4 lg + i: channel kperm(p)
    {
      const float *ip = nullptr;
      if (cd.init_idx >= 0)
        ip = init + ((int64_t)cd.init_idx * H + h) * (kD * kD);
      else if (cd.init_idx <= -2)
        ip = sin + ((int64_t)(-2 - cd.init_idx) * H + h) * (kD * kD);
#pragma unroll
      for (int c = 0; c < NCT; ++c)
#pragma unroll
        for (int ct = 0; ct < 8; ++ct)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            S[c][ct][i] = ip ? ip[kperm(16 * ct + 4 * lg + i) * kD + wcol + 16 * c] : 0.f;
    }
    uint8_t *svw = reinterpret_cast<uint8_t *>(&sm.sv[wv][0]);
    // rows 0..63 of this wave's VW columns of one chunk into its LDS slice:
    // lane l of instruction j moves 16 bytes (8 columns) of row
    // (64 j + l) / (2 NCT); rows past the chunk end read as 0
    auto v_to_lds = [&](int chunk) {
      const int clen = min(kC, cd.ntok - chunk * kC);
      const bf16 *vb =
          v + (cd.tok0 + (int64_t)chunk * kC) * rowstride + (int64_t)h * kD + col0 + VW * wv;
      const __amdgpu_buffer_rsrc_t rv =
          buffer_rsrc(vb, (uint32_t)(((clen - 1) * rowstride + VW) * sizeof(bf16)));
#pragma unroll
      for (int j = 0; j < 2 * NCT; ++j) {
        const int u = 64 * j + lane, r = u / (2 * NCT), qq = u % (2 * NCT);
        lds_load16(rv, (int)((r * rowstride + 8 * qq) * sizeof(bf16)), svw + 1024 * j);
      }
    };
    f32x4 W[NCT][4], Oa[NCT][4]; // of the chunk whose record is current

    // W = K_decay S and O = Q_decay S (K = channels)
    auto stage_wo = [&]() {
      const int ln = opaque_lane(), lr = ln & 15, lg = ln >> 4;
      auto frag = [&](const bf16 *base, int ld, int tile, int s) {
        return load_frag(base + (16 * tile + lr) * ld + 32 * s + 8 * lg);
      };
      Frag<bf16> bs[NCT][4];
#pragma unroll
      for (int c = 0; c < NCT; ++c)
#pragma unroll
        for (int s = 0; s < 4; ++s)
          bs[c][s] = pack_acc2(S[c][2 * s], S[c][2 * s + 1]);
#pragma unroll
      for (int c = 0; c < NCT; ++c)
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
          W[c][tt] = f32x4{0.f, 0.f, 0.f, 0.f};
          Oa[c][tt] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        Frag<bf16> ak[4], aq[4];
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
          ak[tt] = frag(&sm.Kd[0][0], kLdD, tt, s);
          aq[tt] = frag(&sm.Qd[0][0], kLdD, tt, s);
        }
#pragma unroll
        for (int tt = 0; tt < 4; ++tt)
#pragma unroll
          for (int c = 0; c < NCT; ++c) {
            mma(W[c][tt], ak[tt], bs[c][s]);
            mma(Oa[c][tt], aq[tt], bs[c][s]);
          }
      }
    };

    // U = INV Diag(beta) (V - W), O += M_qk U and store o, for chunk ch;
    // U is left packed in bu for the state update
    Frag<bf16> bu[NCT][2];
    // O of chunk ch to o; with the output norm and gate ("Kimi K3.1 Pro 架构完全拆解"
    // §3.3) once the state waves' partial sums are in LDS:
    //   o = sigmoid(gate) w o / sqrt(mean(o^2) + eps) per token row
    auto store_o = [&](int ch) {
      const int ln = opaque_lane(), lr = ln & 15, lg = ln >> 4;
      const int wcol = col0 + VW * wv + lr;
      const int len = min(kC, cd.ntok - ch * kC);
      const int64_t tok = cd.tok0 + (int64_t)ch * kC;
      if constexpr (EPI) {
        float tot = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w)
          tot += sm.Red[w][ln];
        sm.Scl[wv][ln] = __builtin_amdgcn_rsqf(tot * (1.f / kD) + oeps);
        wave_lds_fence();
        // one 16-column tile at a time (fewer live registers)
        const __amdgpu_buffer_rsrc_t rg = buffer_rsrc(
            ogate + tok * rowstride + (int64_t)h * kD, (uint32_t)((len - 1) * rowstride + kD) * 2);
        const int go = (int)((4 * lg * rowstride + wcol) * 2);
#pragma unroll
        for (int c = 0; c < NCT; ++c) {
          float gz[4][4];
#pragma unroll
          for (int tt = 0; tt < 4; ++tt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              gz[tt][i] = buffer_load1(rg, go + (int)((16 * tt + i) * rowstride * 2) + 32 * c,
                                       (const bf16 *)nullptr);
          const float wn = onw ? onw[wcol + 16 * c] : 1.f;
#pragma unroll
          for (int tt = 0; tt < 4; ++tt) {
            const f32x4 sc = *reinterpret_cast<const f32x4 *>(&sm.Scl[wv][16 * tt + 4 * lg]);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const float sg =
                  __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-gz[tt][i] * kLog2e));
              Oa[c][tt][i] *= sc[i] * wn * sg;
            }
          }
        }
      }
      // rows past the chunk end fall outside the buffer and are dropped
      const __amdgpu_buffer_rsrc_t ro = buffer_rsrc(
          o + tok * rowstride + (int64_t)h * kD, (uint32_t)((len - 1) * rowstride + kD) * 2);
      const int vo = (int)((4 * lg * rowstride + wcol) * 2);
#pragma unroll
      for (int tt = 0; tt < 4; ++tt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int so = (int)((16 * tt + i) * rowstride * 2); // wave-uniform
#pragma unroll
          for (int c = 0; c < NCT; ++c)
            buffer_store(ro, static_cast<bf16>(Oa[c][tt][i]), vo + 32 * c, so);
        }
    };

    auto stage_u = [&](int ch) {
      const int ln = opaque_lane(), lr = ln & 15, lg = ln >> 4;
      const int wcol = col0 + VW * wv + lr;
      auto frag = [&](const bf16 *base, int ld, int tile, int s) {
        return load_frag(base + (16 * tile + lr) * ld + 32 * s + 8 * lg);
      };
      const int len = min(kC, cd.ntok - ch * kC);
      const int64_t tok = cd.tok0 + (int64_t)ch * kC;
      wait_vmem_all(); // this chunk's v is in the wave's LDS slice
      const bf16 *svb = &sm.sv[wv][0];
#pragma unroll
      for (int c = 0; c < NCT; ++c)
#pragma unroll
        for (int tt = 0; tt < 4; ++tt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int row = 16 * tt + 4 * lg + i;
            W[c][tt][i] = static_cast<float>(svb[row * VW + 16 * c + lr]) - W[c][tt][i];
          }
      if (ch + 1 < nch) {
        __builtin_amdgcn_s_waitcnt(0xc07f); // lgkmcnt(0): the slice reads have returned
        v_to_lds(ch + 1);
      }
      Frag<bf16> bw[NCT][2];
#pragma unroll
      for (int c = 0; c < NCT; ++c)
#pragma unroll
        for (int s = 0; s < 2; ++s)
          bw[c][s] = pack_acc2(W[c][2 * s], W[c][2 * s + 1]);
      f32x4 U[NCT][4];
#pragma unroll
      for (int c = 0; c < NCT; ++c)
#pragma unroll
        for (int tt = 0; tt < 4; ++tt)
          U[c][tt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        Frag<bf16> ai[4];
#pragma unroll
        for (int tt = 0; tt < 4; ++tt)
          ai[tt] = frag(&sm.INVb[0][0], kLdC, tt, s);
#pragma unroll
        for (int tt = 0; tt < 4; ++tt)
#pragma unroll
          for (int c = 0; c < NCT; ++c)
            mma(U[c][tt], ai[tt], bw[c][s]);
      }
#pragma unroll
      for (int c = 0; c < NCT; ++c)
#pragma unroll
        for (int s = 0; s < 2; ++s)
          bu[c][s] = pack_acc2(U[c][2 * s], U[c][2 * s + 1]);
      // O += M_qk U
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        Frag<bf16> am[4];
#pragma unroll
        for (int tt = 0; tt < 4; ++tt)
          am[tt] = frag(&sm.Mqk[0][0], kLdC, tt, s);
#pragma unroll
        for (int tt = 0; tt < 4; ++tt)
#pragma unroll
          for (int c = 0; c < NCT; ++c)
            mma(Oa[c][tt], am[tt], bu[c][s]);
      }
      if constexpr (EPI) {
        // output norm: this wave's sums of o^2 per token, reduce-scattered
        // over the 16 lanes of a row group (lane lr ends with row tile
        // lr / 4, row lr % 4), to LDS; o leaves after the next barrier
        float x[16];
#pragma unroll
        for (int tt = 0; tt < 4; ++tt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float a = 0.f;
#pragma unroll
            for (int c = 0; c < NCT; ++c)
              a += Oa[c][tt][i] * Oa[c][tt][i];
            x[4 * tt + i] = a;
          }
#pragma unroll
        for (int st = 8; st >= 1; st >>= 1) {
          const bool up = (lr & st) != 0;
#pragma unroll
          for (int m = 0; m < st; ++m) {
            const float send = up ? x[m] : x[m + st];
            const float keep = up ? x[m + st] : x[m];
            x[m] = keep + __shfl_xor(send, st);
          }
        }
        sm.Red[wv][16 * (lr >> 2) + 4 * lg + (lr & 3)] = x[0];
      } else {
        store_o(ch);
      }
    };

    // S = Diag(a_last) S + K_restore^T U (K = tokens), for the chunk whose
    // U was packed into bu by stage_u
    auto stage_s = [&]() {
      const int ln = opaque_lane(), lr = ln & 15, lg = ln >> 4;
      auto frag = [&](const bf16 *base, int ld, int tile, int s) {
        return load_frag(base + (16 * tile + lr) * ld + 32 * s + 8 * lg);
      };
#pragma unroll
      for (int ct = 0; ct < 8; ++ct) {
        const f32x4 a4 = *reinterpret_cast<const f32x4 *>(&sm.aL[16 * ct + 4 * lg]);
#pragma unroll
        for (int c = 0; c < NCT; ++c)
          S[c][ct] *= a4;
      }
#pragma unroll
      for (int s = 0; s < 2; ++s) {
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          Frag<bf16> ar[4];
#pragma unroll
          for (int ct = 0; ct < 4; ++ct)
            ar[ct] = frag(&sm.KrT[0][0], kLdC, 4 * hf + ct, s);
#pragma unroll
          for (int ct = 0; ct < 4; ++ct)
#pragma unroll
            for (int c = 0; c < NCT; ++c)
              mma(S[c][4 * hf + ct], ar[ct], bu[c][s]);
        }
      }
    };

    // the state after chunk ch, when it is one of the chain's checkpoints
    // (the next one is chunk ck_next, at index ck_idx)
    int ck_next = cd.ckpt_chunk, ck_idx = cd.ckpt_idx;
    auto ckpt_store = [&](int ch) {
      if (ckpt != nullptr && ch == ck_next && ch <= cd.ckpt_last) {
        const int ln = opaque_lane(), lr = ln & 15, lg = ln >> 4;
        const int wcol = col0 + VW * wv + lr;
        float *cp = ckpt + ((int64_t)ck_idx * H + h) * (kD * kD);
        ck_next += cd.ckpt_every;
        ++ck_idx;
#pragma unroll
        for (int c = 0; c < NCT; ++c)
#pragma unroll
          for (int ct = 0; ct < 8; ++ct)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              cp[kperm(16 * ct + 4 * lg + i) * kD + wcol + 16 * c] = S[c][ct][i];
      }
    };

    // D_b^-1 = (I - N)(I + N^2)(I + N^4)(I + N^8) for N = L_bb (N^16 = 0), b =
    // this wave's index: the diagonal blocks of INV = (I + L)^-1 of the chunk
    // being prepared, to LDS (for the prep's off-diagonal blocks) and to the
    // record as INV Diag(beta)
    auto stage_inv = [&]() {
      const int ln = opaque_lane(), lr = ln & 15, lg = ln >> 4;
      const int b = wv;
      const float *N = &sm.L[16 * b][16 * b];
      float *P2 = &sm.x.Pow[b][0][0][0];
      float *P4 = &sm.x.Pow[b][1][0][0];
      const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
      const f32x4 n1 = acc_load(N, kLdL, lr, lg);
      f32x4 n2 = zero, n4 = zero, y = zero;
      mm16_lds_acc(n2, N, kLdL, n1, lr, lg); // N^2
      acc_store(P2, kLdB, n2, lr, lg);
      wave_lds_fence();
      mm16_lds_acc(n4, P2, kLdB, n2, lr, lg); // N^4
      acc_store(P4, kLdB, n4, lr, lg);
      wave_lds_fence();
      mm16_lds_acc(y, P4, kLdB, n4, lr, lg); // N^8
#pragma unroll
      for (int i = 0; i < 4; ++i)
        y[i] += (4 * lg + i == lr) ? 1.f : 0.f; // I + N^8
      mm16_lds_acc(y, P4, kLdB, y, lr, lg);      // (I + N^4) Y
      mm16_lds_acc(y, P2, kLdB, y, lr, lg);      // (I + N^2) Y
      mm16_lds_acc(y, N, kLdL, y, lr, lg, -1.f); // (I - N) Y
      acc_store(&sm.Dinv[b][0][0], kLdB, y, lr, lg);
      const float bcol = sm.Beta[16 * b + lr];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        sm.INVb[16 * b + 4 * lg + i][kperm(16 * b + lr)] = static_cast<bf16>(y[i] * bcol);
    };

    // chunk steps 0 .. nch, four barriers each (the ends of stages A-D):
    // step it finishes chunk it - 1 in stages A and B, inverts the diagonal
    // blocks of chunk it in stage C and starts chunk it in stage D
    if (nch == 0) {
      for (int b = 0; b < 4; ++b)
        lds_barrier();
    } else {
      v_to_lds(0);
      lds_barrier();
      lds_barrier();
      stage_inv();
      lds_barrier();
      stage_wo();
      lds_barrier();
      for (int ch = 0; ch + 1 < nch; ++ch) {
        stage_u(ch);
        lds_barrier();
        if constexpr (EPI)
          store_o(ch);
        stage_s();
        ckpt_store(ch);
        lds_barrier();
        stage_inv();
        lds_barrier();
        stage_wo();
        lds_barrier();
      }
      stage_u(nch - 1);
      lds_barrier();
      if constexpr (EPI)
        store_o(nch - 1);
      stage_s();
      ckpt_store(nch - 1);
      lds_barrier();
      lds_barrier();
      lds_barrier();
    }
    if (cd.final_idx >= 0) {
      float *fp = final_state + ((int64_t)cd.final_idx * H + h) * (kD * kD);
#pragma unroll
      for (int c = 0; c < NCT; ++c)
#pragma unroll
        for (int ct = 0; ct < 8; ++ct)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            fp[kperm(16 * ct + 4 * lg + i) * kD + wcol + 16 * c] = S[c][ct][i];
    }
  } else {
    // ============================ prep waves ============================
    const int pw = wv - 4; // token tile
    // raw inputs of the chunk being prepared: channels 32 s + 8 lg .. + 7 of
    // this lane's token, per k-step s
    u32x4 rg[4], rq[4], rk[4];
    // beta stays raw until it is used: widening it where it is loaded would
    // make the wave wait for every load in flight
    unsigned short rbeta = 0;
    auto issue = [&](int chunk) {
      const int ln = opaque_lane(), lr = ln & 15, lg = ln >> 4, r = 16 * pw + lr;
      const int len = min(kC, cd.ntok - chunk * kC);
      const int64_t tok = cd.tok0 + (int64_t)chunk * kC;
      const int64_t base = tok * rowstride + (int64_t)h * kD;
      const uint32_t nbytes = (uint32_t)(((len - 1) * rowstride + kD) * 2);
      const __amdgpu_buffer_rsrc_t bg = buffer_rsrc(g + base, nbytes);
      const __amdgpu_buffer_rsrc_t bk = buffer_rsrc(k + base, nbytes);
      const __amdgpu_buffer_rsrc_t bq = buffer_rsrc(q + base, nbytes);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int vo = (int)((r * rowstride + 32 * s + 8 * lg) * 2);
        rg[s] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(bg, vo, 0, 0));
        rk[s] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(bk, vo, 0, 0));
        rq[s] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(bq, vo, 0, 0));
      }
      if (lg == 0) {
        const __amdgpu_buffer_rsrc_t bb =
            buffer_rsrc(beta + tok * H + h, (uint32_t)(((len - 1) * (int64_t)H + 1) * 2));
        rbeta = __builtin_amdgcn_raw_buffer_load_b16(bb, (int)(r * H * 2), 0, 0);
      }
    };
    if (nch > 0)
      issue(0);
    // prologue: the head's gate scale e^{A_h}
    const bool gate_on = PRO && A_log != nullptr, qk_on = PRO && qk_eps > 0.f;
    const float ea = gate_on ? __expf(A_log[h]) : 1.f;

    float xg[4][8];            // G_loc log2(e) per record channel
    Frag<bf16> fq[4], fk[4];   // Q_loc, K_loc fragments
    f32x4 accLd, accMd;        // diagonal tile pair (L, M_qk)
    f32x4 accLp[2], accMp[2];  // this wave's off-diagonal pairs
    Frag<bf16> kr[4];          // K_restore of this lane's token, record order
    float aLr[2] = {0.f, 0.f}; // a_last of two channels (wave 0)

    for (int it = 0; it < nch; ++it) {
      // ---- stage A: tile scan, Q_loc / K_loc / K_start, diagonal tile pair ----
      {
        const int lane = opaque_lane(), lr = lane & 15, lg = lane >> 4, r = 16 * pw + lr;
        // inclusive cumulative sum over the tile's tokens, then the tile
        // totals (lane 15 of each row) to LDS
        float iq = 1.f, ik = 1.f; // 1 / |q|, 1 / |k| of this lane's token
        if (qk_on) {
          // the token's 128 channels sit in lanes lr, lr + 16, lr + 32, lr + 48
          float sq = 0.f, sk = 0.f;
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            sq = sumsq8_bf16(rq[s], sq);
            sk = sumsq8_bf16(rk[s], sk);
          }
          sq += __shfl_xor(sq, 16);
          sk += __shfl_xor(sk, 16);
          sq += __shfl_xor(sq, 32);
          sk += __shfl_xor(sk, 32);
          iq = __builtin_amdgcn_rsqf(sq + qk_eps);
          ik = __builtin_amdgcn_rsqf(sk + qk_eps);
          if (lg == 0) {
            sm.Iq[r] = iq;
            sm.Ik[r] = ik;
          }
        }
        float G[4][8];
#pragma unroll
        for (int s = 0; s < 4; ++s)
          widen8(rg[s], G[s]);
        if (gate_on) {
          // rows past the chunk end decay by nothing
          const bool valid = r < min(kC, cd.ntok - it * kC);
#pragma unroll
          for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int j = 0; j < 8; ++j)
              G[s][j] = valid ? gate_log_decay(G[s][j], ea, g_min) : 0.f;
        }
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
          for (int j = 0; j < 8; ++j)
            G[s][j] = row_scan16(G[s][j]);
        if (lr == 15) {
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            *reinterpret_cast<f32x4 *>(&sm.Tot[pw][32 * s + 8 * lg]) =
                f32x4{G[s][0], G[s][1], G[s][2], G[s][3]};
            *reinterpret_cast<f32x4 *>(&sm.Tot[pw][32 * s + 8 * lg + 4]) =
                f32x4{G[s][4], G[s][5], G[s][6], G[s][7]};
          }
        }
        if (lg == 0)
          sm.Beta[r] = __builtin_bit_cast(float, (unsigned)rbeta << 16);
        accLd = f32x4{0.f, 0.f, 0.f, 0.f};
        accMd = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          float qv[8], kv[8], xq[8], xk[8], xs[8];
          widen8(rq[s], qv);
          widen8(rk[s], kv);
          if (qk_on) {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
              qv[j] *= iq;
              kv[j] *= ik;
            }
          }
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const float x = G[s][j] * kLog2e;
            xg[s][j] = x;
            const float e1 = __builtin_amdgcn_exp2f(x);
            xq[j] = qv[j] * e1;
            xk[j] = kv[j] * e1;
            xs[j] = kv[j] * __builtin_amdgcn_exp2f(-x);
          }
          fq[s] = pack8(xq);
          fk[s] = pack8(xk);
          const Frag<bf16> fs = pack8(xs);
          *reinterpret_cast<bf16x8 *>(&sm.x.ab.Kst[pw][lr][32 * s + 8 * lg]) = fs.v;
          if (pw == 3) {
            *reinterpret_cast<bf16x8 *>(&sm.x.ab.Aq3[0][lr][32 * s + 8 * lg]) = fk[s].v;
            *reinterpret_cast<bf16x8 *>(&sm.x.ab.Aq3[1][lr][32 * s + 8 * lg]) = fq[s].v;
          }
          mma(accLd, fk[s], fs);
          mma(accMd, fq[s], fs);
        }
        // the diagonal L tile (beta-scaled rows, strictly lower) for the
        // state waves' inversion of the diagonal blocks in stage C
        wave_lds_fence(); // this wave's beta entries are in LDS
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = 16 * pw + 4 * lg + i, col = 16 * pw + lr;
          sm.L[row][col] = col < row ? sm.Beta[row] * accLd[i] : 0.f;
        }
      }
      lds_barrier();
      // ---- stage B: factors, Q_decay / K_decay / K_restore, off-diagonal pairs ----
      {
        const int lane = opaque_lane(), lr = lane & 15, lg = lane >> 4, r = 16 * pw + lr;
        {
          // this tile's factors for two record-order channels per lane
          const int c0 = 2 * lane;
          float t[4][2];
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            const float2 x = *reinterpret_cast<const float2 *>(&sm.Tot[w][c0]);
            t[w][0] = x.x;
            t[w][1] = x.y;
          }
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            float pI = 0.f, gc = 0.f;
#pragma unroll
            for (int w = 0; w < 4; ++w) {
              pI += w < pw ? t[w][e] : 0.f;
              gc += t[w][e];
            }
            sm.Fac[pw][0][c0 + e] = pI * kLog2e;
            sm.Fac[pw][1][c0 + e] = (gc - pI) * kLog2e;
#pragma unroll
            for (int n = 0; n < 2; ++n) {
              if (n < pair_count(pw)) {
                const int I = pair_I(pw, n), J = pair_J(pw, n);
                float sum = 0.f; // p_I - p_J = t_J + ... + t_{I-1} <= 0
#pragma unroll
                for (int w = 0; w < 3; ++w)
                  sum += (w >= J && w < I) ? t[w][e] : 0.f;
                sm.Foff[off_pair(I, J)][c0 + e] = __builtin_amdgcn_exp2f(sum * kLog2e);
              }
            }
            if (pw == 0)
              aLr[e] = __builtin_amdgcn_exp2f(gc * kLog2e);
          }
        }
        wave_lds_fence();
        // Q_decay and K_decay rows to the record, K_restore to registers
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          float xp[8], xc[8], qv[8], kv[8], yq[8], yk[8], yr[8];
          load8f(&sm.Fac[pw][0][32 * s + 8 * lg], xp);
          load8f(&sm.Fac[pw][1][32 * s + 8 * lg], xc);
          widen8(rq[s], qv);
          widen8(rk[s], kv);
          if (qk_on) {
            const float iq = sm.Iq[r], ik = sm.Ik[r];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
              qv[j] *= iq;
              kv[j] *= ik;
            }
          }
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const float a = __builtin_amdgcn_exp2f(xg[s][j] + xp[j]); // e^{G}
            const float b = __builtin_amdgcn_exp2f(xc[j] - xg[s][j]); // e^{G_C - G}
            yq[j] = qv[j] * a;
            yk[j] = kv[j] * a;
            yr[j] = kv[j] * b;
          }
          *reinterpret_cast<bf16x8 *>(&sm.Qd[r][32 * s + 8 * lg]) = pack8(yq).v;
          *reinterpret_cast<bf16x8 *>(&sm.Kd[r][32 * s + 8 * lg]) = pack8(yk).v;
          kr[s] = pack8(yr);
        }
        // off-diagonal pairs (I, J): B = K_start of tile J times e^{p_I - p_J}
#pragma unroll
        for (int n = 0; n < 2; ++n) {
          accLp[n] = f32x4{0.f, 0.f, 0.f, 0.f};
          accMp[n] = f32x4{0.f, 0.f, 0.f, 0.f};
          if (n < pair_count(pw)) {
            const int I = pair_I(pw, n), J = pair_J(pw, n);
            const int pi = off_pair(I, J);
#pragma unroll
            for (int s = 0; s < 4; ++s) {
              const Frag<bf16> e = load_frag(&sm.x.ab.Kst[J][lr][32 * s + 8 * lg]);
              float xs[8], fo[8];
              frag_to_f32(e, xs);
              load8f(&sm.Foff[pi][32 * s + 8 * lg], fo);
#pragma unroll
              for (int j = 0; j < 8; ++j)
                xs[j] *= fo[j];
              const Frag<bf16> b = pack8(xs);
              Frag<bf16> ak, aq;
              if (I == pw) {
                ak = fk[s];
                aq = fq[s];
              } else {
                ak = load_frag(&sm.x.ab.Aq3[0][lr][32 * s + 8 * lg]);
                aq = load_frag(&sm.x.ab.Aq3[1][lr][32 * s + 8 * lg]);
              }
              mma(accLp[n], ak, b);
              mma(accMp[n], aq, b);
            }
          }
        }
        // the next chunk's inputs are in flight from here on
        if (it + 1 < nch)
          issue(it + 1);
      }
      lds_barrier();
      // ---- stage C: L / M_qk tiles, K_restore^T, a_last -------------------------
      {
        const int lane = opaque_lane(), lr = lane & 15, lg = lane >> 4, r = 16 * pw + lr;
        // off-diagonal tiles (I > J: no mask) and the diagonal M_qk tile
#pragma unroll
        for (int n = 0; n < 2; ++n)
          if (n < pair_count(pw)) {
            const int I = pair_I(pw, n), J = pair_J(pw, n), col = 16 * J + lr;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int row = 16 * I + 4 * lg + i;
              sm.L[row][col] = sm.Beta[row] * accLp[n][i];
              sm.Mqk[row][kperm(col)] = static_cast<bf16>(accMp[n][i]);
            }
          }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = 16 * pw + 4 * lg + i, col = 16 * pw + lr;
          sm.Mqk[row][kperm(col)] = static_cast<bf16>(col <= row ? accMd[i] : 0.f);
        }
        // K_restore^T: row kperm_inv(channel), column kperm(token)
        {
          const int kc = kperm(r);
#pragma unroll
          for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int e = 0; e < 8; ++e)
              sm.KrT[kperm_inv(32 * s + 8 * lg + e)][kc] = kr[s].v[e];
        }
        if (pw == 0) {
          sm.aL[kperm_inv(2 * lane)] = aLr[0];
          sm.aL[kperm_inv(2 * lane + 1)] = aLr[1];
        }
      }
      lds_barrier();
      // ---- stage D: off-diagonal blocks of INV ---------------------------------
      {
        const int lane = opaque_lane(), lr = lane & 15, lg = lane >> 4;
        // column block j = pw: X_ij = -D_i^-1 sum_{m=j}^{i-1} L_im X_mj
        const int j = pw;
        const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
        f32x4 X[4];
        const f32x4 dj = acc_load(&sm.Dinv[j][0][0], kLdB, lr, lg);
#pragma unroll
        for (int t = 0; t < 4; ++t)
          X[t] = (t == j) ? dj : zero;
        const float bcol = sm.Beta[16 * j + lr];
#pragma unroll
        for (int i = 1; i < 4; ++i) {
          if (i > j) {
            f32x4 t = zero;
#pragma unroll
            for (int m = 0; m < 3; ++m)
              if (m >= j && m < i)
                mm16_lds_acc(t, &sm.L[16 * i][16 * m], kLdL, X[m], lr, lg);
            f32x4 x = zero;
            mm16_lds_acc(x, &sm.Dinv[i][0][0], kLdB, t, lr, lg, -1.f);
            X[i] = x;
#pragma unroll
            for (int e = 0; e < 4; ++e)
              sm.INVb[16 * i + 4 * lg + e][kperm(16 * j + lr)] = static_cast<bf16>(x[e] * bcol);
          }
        }
      }
      lds_barrier();
    }
    // the last chunk step only consumes the last record
    for (int b = 0; b < 4; ++b)
      lds_barrier();
  }
}

hipError_t launch_fused(const ChainDesc *chains, int32_t nchains, int32_t H, const void *q,
                        const void *k, const void *v, const void *g, const void *beta, void *o,
                        const float *init, const float *sin, float *final_state, float *ckpt,
                        const Prologue &pro, const Epilogue &epi, hipStream_t s) {
  if (nchains == 0)
    return hipSuccess;
  // one workgroup per (chain, head) carries all 128 state columns
  constexpr int NCT = 2;
  dim3 grid((unsigned)nchains, (unsigned)H, kD / (64 * NCT)), block(kFThreads);
  auto launch = [&](auto kern) {
    kern<<<grid, block, 0, s>>>(chains, H, (const bf16 *)q, (const bf16 *)k, (const bf16 *)v,
                                (const bf16 *)g, (const bf16 *)beta, (bf16 *)o, init, sin,
                                final_state, ckpt, pro.A_log, pro.g_min, pro.qk_eps,
                                (const bf16 *)epi.gate, epi.weight, epi.eps);
  };
  if (epi.on())
    launch(fused_kernel<NCT, true, true>);
  else if (pro.on())
    launch(fused_kernel<NCT, true, false>);
  else
    launch(fused_kernel<NCT, false, false>);
  return hipGetLastError();
}

} // namespace kda
