// KDA chunked prefill, chunk prep and state carry fused in one kernel (bf16).
//
// Same mathematics as the two-kernel path (kda_prefill.hip): the FlashKDA
// chunk form of "Kimi K3 的架構" (hao.cnyes.com) §六 with the 16-token
// reference points that the decay's lower bound allows ("Kimi K3.1 Pro
// 架构完全拆解" §3.2).  The difference is where the chunk-prep results live:
// here they never leave the compute unit.
//
// One workgroup of 8 waves owns one (chain, head, 64-column block of S):
//   waves 0-3 ("state") walk the chunks in order and keep their 128 x 64 slice
//   of S in MFMA accumulators:  W = K_decay S,  U = INV Diag(beta)(V - W),
//   O = Q_decay S + M_qk U,  S = Diag(a_last) S + K_restore^T U;
//   waves 4-7 ("prep") build the operands of the NEXT chunk meanwhile:
//   cumulative log-decay, decayed q/k, L and M_qk on MFMA, INV = (I + L)^-1.
// The prep results pass to the state waves through LDS ("hand-off" arrays);
// a chunk's q, k, g and beta are loaded one chunk before the prep needs them,
// and v one chunk before the state needs it.  Per chunk the only HBM traffic
// is the layer's own inputs and outputs.
//
// Prep lane layout: prep wave pw owns token tile pw (rows 16pw .. 16pw+15);
// lane (lr, lg) holds row 16pw + lr and channels 32s + 8lg .. +7 for
// s = 0..3, which is exactly the MFMA fragment layout, so the decayed
// operands of the L / M_qk products are built in registers.  The cumulative
// sum over rows inside a tile is a DPP scan across the 16 lanes of a row.
//
// Numerics (log-decay kept in log2 units, g * log2(e)):
//   G_loc  = inclusive cumsum of g inside the 16-token tile, in (-80/ln2, 0]
//   p_I    = cumulative log-decay before tile I,  p_4 = whole chunk
//   K_loc  = k 2^{G_loc},  Q_loc = q 2^{G_loc}          (A side, <= 1)
//   K_st   = k 2^{-G_loc}                               (diagonal B, <= e^80)
//   K_end  = K_st 2^{p_{I+1} - p_I}                     (<= 1)
//   B(I,J) = K_end(J) 2^{p_I - p_{J+1}}  for J < I       (<= 1)
//   K_decay = K_loc 2^{p_I},  Q_decay = Q_loc 2^{p_I},  K_restore = K_end 2^{p_4 - p_{I+1}}
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

namespace {

constexpr int kFThreads = 512;
constexpr int kFBV = 64;           // state columns per workgroup
constexpr int kNCT = kFBV / 16;    // 16-column tiles of the state slice
constexpr int kLdD = kD + 8;       // padded row length, 128-wide bf16 arrays
constexpr int kLdC = kC + 8;       // padded row length, 64-wide bf16 arrays
constexpr int kLdL = kC + 4;       // padded row length, fp32 L / INV (16-byte rows)
constexpr int kLdB = 20;           // padded row length, fp32 16 x 16 blocks (16-byte rows)
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kStagesPerChunk = 5; // barriers per chunk, identical in both roles

struct FusedSmem {
  // state working set; Sb's bytes also hold the fp32 L / D^-1 matrix while
  // the prep inverts it (the state waves do not touch Sb then)
  bf16 Sb[kFBV][kLdD];
  bf16 VWb[kFBV][kLdC];
  bf16 Ub[kFBV][kLdC];
  // hand-off, prep -> state
  bf16 hKd[kC][kLdD];
  bf16 hQd[kC][kLdD];
  bf16 hKrT[kD][kLdC];
  bf16 hINVb[kC][kLdC];
  bf16 hMqk[kC][kLdC];
  float hAc[kD];
  // prep working set
  bf16 sKe[kC][kLdD];
  float sTot[4][kD];
  float sEp[4][kD], sEs[4][kD], sEr[4][kD];
  float sF[6][kD];
  float sBeta[kC];
  float sD[4][16][kLdB];      // D_b^-1, the inverted diagonal blocks of I + L
  float sPow[4][2][16][kLdB]; // per prep wave: N^2 and N^4 of its diagonal block
};
static_assert(sizeof(FusedSmem) <= 160 * 1024, "LDS budget");
static_assert(sizeof(float) * kC * kLdL <= sizeof(bf16) * kFBV * kLdD, "L fits in Sb");

// off-diagonal tile pairs (I > J): index of exp(p_I - p_{J+1}) in sF
__device__ __forceinline__ int off_pair(int I, int J) {
  // (1,0)->0 (2,0)->1 (2,1)->2 (3,0)->3 (3,1)->4 (3,2)->5
  return (I * (I - 1)) / 2 + J;
}

// Lane index as an opaque value: the compiler cannot hoist lane-dependent
// address arithmetic built on it out of the chunk loop, which would keep
// dozens of loop-invariant LDS addresses alive in registers across stages.
__device__ __forceinline__ int opaque_lane() {
  int l;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return l;
}

// Stage boundary: LDS-ordering barrier that the instruction scheduler may
// not move work across (each stage's register live ranges stay inside it).
__device__ __forceinline__ void fsync() {
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
  __builtin_amdgcn_sched_barrier(0);
}

__device__ __forceinline__ float dpp_shr(float x, int n) {
  int v = __builtin_bit_cast(int, x);
  int r;
  switch (n) {
  case 1: r = __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, true); break;
  case 2: r = __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, true); break;
  case 4: r = __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, true); break;
  default: r = __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, true); break;
  }
  return __builtin_bit_cast(float, r);
}

// Inclusive prefix sum over the 16 lanes of each DPP row (row_shr with
// bound_ctrl: lanes before the row start read 0).
__device__ __forceinline__ float row_scan16(float x) {
  x += dpp_shr(x, 1);
  x += dpp_shr(x, 2);
  x += dpp_shr(x, 4);
  x += dpp_shr(x, 8);
  return x;
}

// Raw inputs of one chunk, in the prep lane layout.
struct PrepRaw {
  bf16x8 q[4], k[4], g[4];
  float beta;
};

// g and beta (needed first) and q, k (needed two stages later) are loaded
// separately to keep their register live ranges short.
__device__ __forceinline__ void prep_load_g(PrepRaw &raw, const bf16 *g, const bf16 *beta,
                                            int64_t tok0, int len, int H, int h,
                                            int64_t rowstride, int pw, int lr, int lg) {
  const int rr = min(16 * pw + lr, len - 1);
  const int64_t base = (tok0 + rr) * rowstride + (int64_t)h * kD + 8 * lg;
#pragma unroll
  for (int s = 0; s < 4; ++s)
    raw.g[s] = *reinterpret_cast<const bf16x8 *>(g + base + 32 * s);
  raw.beta = static_cast<float>(beta[(tok0 + rr) * H + h]);
}

__device__ __forceinline__ void prep_load_qk(PrepRaw &raw, const bf16 *q, const bf16 *k,
                                             int64_t tok0, int len, int h, int64_t rowstride,
                                             int pw, int lr, int lg) {
  const int rr = min(16 * pw + lr, len - 1);
  const int64_t base = (tok0 + rr) * rowstride + (int64_t)h * kD + 8 * lg;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    raw.k[s] = *reinterpret_cast<const bf16x8 *>(k + base + 32 * s);
    raw.q[s] = *reinterpret_cast<const bf16x8 *>(q + base + 32 * s);
  }
}

} // namespace

// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kFThreads) void fused_kernel(
    const ChainDesc *__restrict__ chains, int32_t H, const bf16 *__restrict__ q,
    const bf16 *__restrict__ k, const bf16 *__restrict__ v, const bf16 *__restrict__ g,
    const bf16 *__restrict__ beta, bf16 *__restrict__ o, const float *__restrict__ init,
    const float *__restrict__ sin, float *__restrict__ final_state) {
  __shared__ __attribute__((aligned(16))) FusedSmem sm;
  float(*sL)[kLdL] = reinterpret_cast<float(*)[kLdL]>(&sm.Sb[0][0]);

  const ChainDesc cd = chains[blockIdx.x];
  const int h = blockIdx.y;
  const int vcol0 = blockIdx.z * kFBV;
  const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63, lr = lane & 15, lg = lane >> 4;
  const int64_t rowstride = (int64_t)H * kD;
  const int nch = (cd.ntok + kC - 1) / kC;

  // zero the upper 16 x 16 blocks of INV*Diag(beta) and M_qk once; the prep
  // only ever writes their lower blocks
  for (int e = tid; e < 6 * 256; e += kFThreads) {
    const int t = e >> 8, r = (e >> 4) & 15, c = e & 15;
    const int bi = t < 3 ? 0 : (t < 5 ? 1 : 2);
    const int bj = t < 3 ? t + 1 : (t < 5 ? t - 1 : 3);
    sm.hINVb[16 * bi + r][16 * bj + c] = static_cast<bf16>(0.f);
    sm.hMqk[16 * bi + r][16 * bj + c] = static_cast<bf16>(0.f);
  }

  const bf16 *vchain = v + cd.tok0 * rowstride + (int64_t)h * kD + vcol0;
  // The role is uniform per wave; readfirstlane makes the branch scalar, so
  // each wave runs exactly one side and both sides pass the same barriers.
  const int wvu = __builtin_amdgcn_readfirstlane(tid >> 6);
  if (wvu < 4) {
    // ===================== state waves =====================
    f32x4 sacc[2][kNCT];
    Frag<bf16> mqk[2], krt[2][2];
    f32x4 acv[2];
    bf16 vcur[kNCT][4], vnxt[kNCT][4];
  auto load_v = [&](bf16 (&dst)[kNCT][4], int chunk) {
      const int len = min(kC, cd.ntok - chunk * kC);
      const bf16 *vb = vchain + (int64_t)chunk * kC * rowstride;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int rr = min(16 * wv + 4 * lg + i, len - 1);
#pragma unroll
        for (int ct = 0; ct < kNCT; ++ct)
          dst[ct][i] = vb[(int64_t)rr * rowstride + 16 * ct + lr];
      }
    };


    {
      const float *ip = nullptr;
      if (cd.init_idx >= 0)
        ip = init + ((int64_t)cd.init_idx * H + h) * (kD * kD);
      else if (cd.init_idx <= -2)
        ip = sin + ((int64_t)(-2 - cd.init_idx) * H + h) * (kD * kD);
#pragma unroll
      for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int ct = 0; ct < kNCT; ++ct)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int row = 16 * (2 * wv + rt) + 4 * lg + i;
            sacc[rt][ct][i] = ip ? ip[row * kD + vcol0 + 16 * ct + lr] : 0.f;
          }
    }
    if (nch > 0) {
      load_v(vcur, 0);
      for (int b = 0; b < kStagesPerChunk; ++b) // the prep builds chunk 0
        fsync();
    }
    for (int ch = 0; ch < nch; ++ch) {
      const int len = min(kC, cd.ntok - ch * kC);
      // ---- stage 1: copy the small hand-off arrays, S -> Sb, prefetch v
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        mqk[s] = load_frag(&sm.hMqk[16 * wv + lr][32 * s + 8 * lg]);
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
          krt[rt][s] = load_frag(&sm.hKrT[16 * (2 * wv + rt) + lr][32 * s + 8 * lg]);
      }
#pragma unroll
      for (int rt = 0; rt < 2; ++rt)
        acv[rt] = *reinterpret_cast<const f32x4 *>(&sm.hAc[16 * (2 * wv + rt) + 4 * lg]);
#pragma unroll
      for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int ct = 0; ct < kNCT; ++ct)
          store4(&sm.Sb[16 * ct + lr][16 * (2 * wv + rt) + 4 * lg], sacc[rt][ct][0],
                 sacc[rt][ct][1], sacc[rt][ct][2], sacc[rt][ct][3]);
      if (ch + 1 < nch)
        load_v(vnxt, ch + 1);
      fsync();
      // ---- stage 2: W = K_decay S, O = Q_decay S, V - W -> VWb
      f32x4 Oa[kNCT];
      {
        f32x4 W[kNCT];
#pragma unroll
        for (int ct = 0; ct < kNCT; ++ct) {
          W[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
          Oa[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const int kb = 32 * s + 8 * lg;
          const Frag<bf16> akd = load_frag(&sm.hKd[16 * wv + lr][kb]);
          const Frag<bf16> aqd = load_frag(&sm.hQd[16 * wv + lr][kb]);
#pragma unroll
          for (int ct = 0; ct < kNCT; ++ct) {
            const Frag<bf16> b = load_frag(&sm.Sb[16 * ct + lr][kb]);
            mma(W[ct], akd, b);
            mma(Oa[ct], aqd, b);
          }
        }
#pragma unroll
        for (int ct = 0; ct < kNCT; ++ct) {
          float x[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int row = 16 * wv + 4 * lg + i;
            const float vv = row < len ? static_cast<float>(vcur[ct][i]) : 0.f;
            x[i] = vv - W[ct][i];
          }
          store4(&sm.VWb[16 * ct + lr][16 * wv + 4 * lg], x[0], x[1], x[2], x[3]);
        }
      }
      fsync();
      // ---- stage 3: U = INV Diag(beta) (V - W) -> Ub
      {
        f32x4 U[kNCT];
#pragma unroll
        for (int ct = 0; ct < kNCT; ++ct)
          U[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const int kb = 32 * s + 8 * lg;
          const Frag<bf16> a = load_frag(&sm.hINVb[16 * wv + lr][kb]);
#pragma unroll
          for (int ct = 0; ct < kNCT; ++ct) {
            const Frag<bf16> b = load_frag(&sm.VWb[16 * ct + lr][kb]);
            mma(U[ct], a, b);
          }
        }
#pragma unroll
        for (int ct = 0; ct < kNCT; ++ct)
          store4(&sm.Ub[16 * ct + lr][16 * wv + 4 * lg], U[ct][0], U[ct][1], U[ct][2],
                 U[ct][3]);
      }
      fsync();
      // ---- stage 4: O = Q_decay S + M_qk U (stored), S = Diag(a) S + K_restore^T U
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const int kb = 32 * s + 8 * lg;
#pragma unroll
        for (int ct = 0; ct < kNCT; ++ct) {
          const Frag<bf16> b = load_frag(&sm.Ub[16 * ct + lr][kb]);
          mma(Oa[ct], mqk[s], b);
        }
      }
      bf16 *orow = o + (cd.tok0 + (int64_t)ch * kC) * rowstride + (int64_t)h * kD + vcol0;
#pragma unroll
      for (int ct = 0; ct < kNCT; ++ct)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = 16 * wv + 4 * lg + i;
          if (row < len)
            orow[(int64_t)row * rowstride + 16 * ct + lr] = static_cast<bf16>(Oa[ct][i]);
        }
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) {
#pragma unroll
        for (int ct = 0; ct < kNCT; ++ct)
          sacc[rt][ct] *= acv[rt];
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const int kb = 32 * s + 8 * lg;
#pragma unroll
          for (int ct = 0; ct < kNCT; ++ct) {
            const Frag<bf16> b = load_frag(&sm.Ub[16 * ct + lr][kb]);
            mma(sacc[rt][ct], krt[rt][s], b);
          }
        }
      }
#pragma unroll
      for (int ct = 0; ct < kNCT; ++ct)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          vcur[ct][i] = vnxt[ct][i];
      fsync();
      // ---- stages 5-7: the prep finishes INV for the next chunk
      for (int b = 4; b < kStagesPerChunk; ++b)
        fsync();
    }
    if (cd.final_idx >= 0) {
      float *fp = final_state + ((int64_t)cd.final_idx * H + h) * (kD * kD);
#pragma unroll
      for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int ct = 0; ct < kNCT; ++ct)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int row = 16 * (2 * wv + rt) + 4 * lg + i;
            fp[row * kD + vcol0 + 16 * ct + lr] = sacc[rt][ct][i];
          }
    }
  } else {
    // ===================== prep waves =====================
    const int pw = wvu - 4;
    PrepRaw raw;
    Frag<bf16> aK[4], aQ[4], bS[4];
    float gl[32];
    f32x4 accL[4], accM[4];
  // The prep pipeline for one chunk, split into the stages that line up with
    // the state waves' stages (every stage ends with a workgroup barrier).
    // Stage P1: cumulative decay inside each tile, tile totals, beta.
    auto prep_scan = [&](int chunk) {
      const int lane_ = opaque_lane(), lr = lane_ & 15, lg = lane_ >> 4;
      const int len = min(kC, cd.ntok - chunk * kC);
      const int r = 16 * pw + lr;
      const bool ok = r < len;
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float x = ok ? static_cast<float>(raw.g[s][j]) * kLog2e : 0.f;
          gl[8 * s + j] = row_scan16(x);
        }
      if (lr == 15) {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          *reinterpret_cast<f32x4 *>(&sm.sTot[pw][32 * s + 8 * lg]) =
              f32x4{gl[8 * s], gl[8 * s + 1], gl[8 * s + 2], gl[8 * s + 3]};
          *reinterpret_cast<f32x4 *>(&sm.sTot[pw][32 * s + 8 * lg + 4]) =
              f32x4{gl[8 * s + 4], gl[8 * s + 5], gl[8 * s + 6], gl[8 * s + 7]};
        }
      }
      if (lg == 0)
        sm.sBeta[r] = ok ? raw.beta : 0.f;
    };
    // Stage P2: per-channel factor tables from the tile totals.
    auto prep_tables = [&]() {
      const int pt = tid - 256;
      const int c = pt & (kD - 1);
      const float t0 = sm.sTot[0][c], t1 = sm.sTot[1][c], t2 = sm.sTot[2][c], t3 = sm.sTot[3][c];
      const float p[5] = {0.f, t0, t0 + t1, t0 + t1 + t2, t0 + t1 + t2 + t3};
      if (pt < 128) {
#pragma unroll
        for (int I = 0; I < 4; ++I) {
          sm.sEp[I][c] = __builtin_amdgcn_exp2f(p[I]);
          sm.sEs[I][c] = __builtin_amdgcn_exp2f(p[I + 1] - p[I]);
        }
        sm.hAc[c] = __builtin_amdgcn_exp2f(p[4]);
      } else {
#pragma unroll
        for (int I = 0; I < 4; ++I)
          sm.sEr[I][c] = __builtin_amdgcn_exp2f(p[4] - p[I + 1]);
        sm.sF[0][c] = __builtin_amdgcn_exp2f(p[1] - p[1]);
        sm.sF[1][c] = __builtin_amdgcn_exp2f(p[2] - p[1]);
        sm.sF[2][c] = __builtin_amdgcn_exp2f(p[2] - p[2]);
        sm.sF[3][c] = __builtin_amdgcn_exp2f(p[3] - p[1]);
        sm.sF[4][c] = __builtin_amdgcn_exp2f(p[3] - p[2]);
        sm.sF[5][c] = __builtin_amdgcn_exp2f(p[3] - p[3]);
      }
    };
    // Stage P3: decayed operands of this lane's row, produced two channels at
    // a time and packed to bf16 at once so few fp32 temporaries are live.
    auto prep_elem = [&](int chunk) {
      const int lane_ = opaque_lane(), lr = lane_ & 15, lg = lane_ >> 4;
      const int len = min(kC, cd.ntok - chunk * kC);
      const int r = 16 * pw + lr;
      const bool ok = r < len;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int c0 = 32 * s + 8 * lg;
        bf16x8 vkl, vql, vks, vke, vkd, vqd;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float kv = ok ? static_cast<float>(raw.k[s][j]) : 0.f;
          const float qv = ok ? static_cast<float>(raw.q[s][j]) : 0.f;
          const float el = __builtin_amdgcn_exp2f(gl[8 * s + j]);   // (e^-80, 1]
          const float es_ = __builtin_amdgcn_exp2f(-gl[8 * s + j]); // [1, e^80)
          const float ep = sm.sEp[pw][c0 + j];
          const float kl = kv * el, ql = qv * el, ks = kv * es_;
          const float ke = ks * sm.sEs[pw][c0 + j];
          vkl[j] = static_cast<bf16>(kl);
          vql[j] = static_cast<bf16>(ql);
          vks[j] = static_cast<bf16>(ks);
          vke[j] = static_cast<bf16>(ke);
          vkd[j] = static_cast<bf16>(kl * ep);
          vqd[j] = static_cast<bf16>(ql * ep);
          // K_restore^T: column r of row c0 + j
          sm.hKrT[c0 + j][r] = static_cast<bf16>(ke * sm.sEr[pw][c0 + j]);
        }
        aK[s].v = vkl;
        aQ[s].v = vql;
        bS[s].v = vks;
        *reinterpret_cast<bf16x8 *>(&sm.sKe[r][c0]) = vke;
        *reinterpret_cast<bf16x8 *>(&sm.hKd[r][c0]) = vkd;
        *reinterpret_cast<bf16x8 *>(&sm.hQd[r][c0]) = vqd;
        // one channel group at a time keeps the temporaries' live ranges short
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    // Stage P4: L and M_qk tiles of row tile pw on MFMA.
    auto prep_mfma = [&]() {
      const int lane_ = opaque_lane(), lr = lane_ & 15, lg = lane_ >> 4;
#pragma unroll
      for (int J = 0; J < 4; ++J) {
        accL[J] = f32x4{0.f, 0.f, 0.f, 0.f};
        accM[J] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (J <= pw) {
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            Frag<bf16> b;
            if (J == pw) {
              b = bS[s];
            } else {
              const int c0 = 32 * s + 8 * lg;
              const Frag<bf16> e = load_frag(&sm.sKe[16 * J + lr][c0]);
              const float *f = &sm.sF[off_pair(pw, J)][c0];
              float x[8];
              frag_to_f32(e, x);
#pragma unroll
              for (int j = 0; j < 8; ++j)
                x[j] *= f[j];
              b = frag_from_f32<bf16>(x);
            }
            mma(accL[J], aK[s], b);
            mma(accM[J], aQ[s], b);
          }
        }
      }
      // M_qk (diagonal kept) to the hand-off; lower tiles only
#pragma unroll
      for (int J = 0; J < 4; ++J) {
        if (J <= pw) {
          const int col = 16 * J + lr;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int row = 16 * pw + 4 * lg + i;
            sm.hMqk[row][col] = static_cast<bf16>(col <= row ? accM[J][i] : 0.f);
          }
        }
      }
    };
    // Stage P5: L = StrictTril(Diag(beta) ...) into the fp32 matrix (in Sb).
    auto prep_store_L = [&]() {
      const int lane_ = opaque_lane(), lr = lane_ & 15, lg = lane_ >> 4;
#pragma unroll
      for (int J = 0; J < 4; ++J) {
        if (J <= pw) {
          const int col = 16 * J + lr;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int row = 16 * pw + 4 * lg + i;
            sL[row][col] = col < row ? sm.sBeta[row] * accL[J][i] : 0.f;
          }
        }
      }
    };
    // INV = (I + L)^-1 by 16 x 16 blocks, all products on fp32 MFMA.
    // Level 0 (wave b, no cross-wave data): D_b = I + N with N = L_bb strictly
    // lower, so D_b^-1 = (I - N)(I + N^2)(I + N^4)(I + N^8) exactly (N^16 = 0).
    // X_bb = D_b^-1 stays in registers as this wave's first block of its
    // column block of INV.
    f32x4 X[4];
    auto inv_level0 = [&]() {
      const int lane_ = opaque_lane(), lr = lane_ & 15, lg = lane_ >> 4;
      const int b = pw;
      const float *N = &sL[16 * b][16 * b];
      float *P2 = &sm.sPow[b][0][0][0];
      float *P4 = &sm.sPow[b][1][0][0];
      const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
      const f32x4 n1 = acc_load(N, kLdL, lr, lg);
      f32x4 n2 = zero, n4 = zero, y = zero;
      mm16_lds_acc(n2, N, kLdL, n1, lr, lg);          // N^2
      acc_store(P2, kLdB, n2, lr, lg);
      mm16_lds_acc(n4, P2, kLdB, n2, lr, lg);         // N^4
      acc_store(P4, kLdB, n4, lr, lg);
      mm16_lds_acc(y, P4, kLdB, n4, lr, lg);          // N^8
#pragma unroll
      for (int i = 0; i < 4; ++i)
        y[i] += (4 * lg + i == lr) ? 1.f : 0.f;        // I + N^8
      mm16_lds_acc(y, P4, kLdB, y, lr, lg);           // (I + N^4) Y
      mm16_lds_acc(y, P2, kLdB, y, lr, lg);           // (I + N^2) Y
      mm16_lds_acc(y, N, kLdL, y, lr, lg, -1.f);      // (I - N) Y
#pragma unroll
      for (int t = 0; t < 4; ++t)
        if (t == b)
          X[t] = y; // static register index
      acc_store(&sm.sD[b][0][0], kLdB, y, lr, lg);
      const float bcol = sm.sBeta[16 * b + lr];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        sm.hINVb[16 * b + 4 * lg + i][16 * b + lr] = static_cast<bf16>(y[i] * bcol);
    };
    // Level 1: wave j walks down its column block of INV by block forward
    // substitution, X_ij = -D_i^-1 sum_{m=j}^{i-1} L_im X_mj, using only its
    // own earlier blocks, the shared L and the D_i^-1 of level 0.
    auto inv_level1 = [&]() {
      const int lane_ = opaque_lane(), lr = lane_ & 15, lg = lane_ >> 4;
      const int j = pw;
      const float bcol = sm.sBeta[16 * j + lr];
#pragma unroll
      for (int i = 1; i < 4; ++i) {
        if (i > j) {
          f32x4 t = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int m = 0; m < 3; ++m)
            if (m >= j && m < i)
              mm16_lds_acc(t, &sL[16 * i][16 * m], kLdL, X[m], lr, lg);
          f32x4 x = {0.f, 0.f, 0.f, 0.f};
          mm16_lds_acc(x, &sm.sD[i][0][0], kLdB, t, lr, lg, -1.f);
          X[i] = x;
#pragma unroll
          for (int r = 0; r < 4; ++r)
            sm.hINVb[16 * i + 4 * lg + r][16 * j + lr] = static_cast<bf16>(x[r] * bcol);
        }
      }
    };

    // One chunk's preparation, in kStagesPerChunk barrier-separated stages.
    // Its raw inputs must already be in `raw`; the next chunk's inputs are
    // loaded as soon as these are consumed.
    auto prep_chunk = [&](int chunk, bool active) {
      const bool more = chunk + 1 < nch;
      const int64_t ntok0 = cd.tok0 + (int64_t)(chunk + 1) * kC;
      const int nlen = min(kC, cd.ntok - (chunk + 1) * kC);
      if (active) prep_scan(chunk);
      fsync();
      if (active) prep_tables();
      fsync();
      if (active) prep_elem(chunk);
      fsync();
      if (more)
        prep_load_g(raw, g, beta, ntok0, nlen, H, h, rowstride, pw, lr, lg);
      if (active) {
        prep_mfma();
        prep_store_L(); // sL rows of tile pw: read below by this wave only
        inv_level0();
      }
      fsync();
      if (more)
        prep_load_qk(raw, q, k, ntok0, nlen, h, rowstride, pw, lr, lg);
      if (active) inv_level1();
      fsync();
    };
    if (nch > 0) {
      prep_load_g(raw, g, beta, cd.tok0, min(kC, cd.ntok), H, h, rowstride, pw, lr, lg);
      prep_load_qk(raw, q, k, cd.tok0, min(kC, cd.ntok), h, rowstride, pw, lr, lg);
      prep_chunk(0, true);
    }
    for (int ch = 0; ch < nch; ++ch)
      prep_chunk(ch + 1, ch + 1 < nch);
  }
}

hipError_t launch_fused(const ChainDesc *chains, int32_t nchains, int32_t H, const void *q,
                        const void *k, const void *v, const void *g, const void *beta, void *o,
                        const float *init, const float *sin, float *final_state,
                        hipStream_t s) {
  if (nchains == 0)
    return hipSuccess;
  dim3 grid((unsigned)nchains, (unsigned)H, kD / kFBV), block(kFThreads);
  fused_kernel<<<grid, block, 0, s>>>(chains, H, (const bf16 *)q, (const bf16 *)k,
                                      (const bf16 *)v, (const bf16 *)g, (const bf16 *)beta,
                                      (bf16 *)o, init, sin, final_state);
  return hipGetLastError();
}

} // namespace kda
