// Causal prefill attention on CDNA4 matrix cores (gfx950) for the V2/V3 head
// shape: q, k [T, H, 192] and v [T, H, 128] in bf16, o [T, H, 128].
//   o[t, h] = sum_{j <= t} softmax_j(scale * q[t,h] . k[j,h]) v[j,h]
// (NeMo "MLA" module: forward with a causal attention mask and softmax_scale).
//
// Flash-style: a workgroup owns 32*NW queries of one head and streams 64-key tiles
// of K and V through three LDS buffers (direct global->LDS buffer copies, two tiles in
// flight, one fence-free barrier per tile).  Each wave
// keeps 32 queries: S^T = K Q^T with keys as the M dimension, so the softmax
// probabilities are already in the B-operand layout of O^T = V^T P^T; V^T is read
// with the transposing LDS read.  Online softmax in the log2 domain with a lazy
// rescale (the running max only moves when a tile exceeds it by 2^8).
// Workgroups are ordered heaviest first (latest query tiles) and grouped so that
// the query tiles of one head run on one XCD and share its L2.
#include "mla_fast.h"

namespace mla {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

constexpr int DQK = 192, DV = 128;
constexpr int KC = DQK / 8, VC = DV / 8;   // 16-byte chunks per key / value row
constexpr int KT = 64;                     // keys per tile
constexpr int K_SLOTS = KT * KC, V_SLOTS = KT * VC;
constexpr float kRescaleThreshold = 8.0f;
constexpr int kXcds = 8;

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

// K tile: key t, chunk c at slot KC*t + (c ^ k_swz(t)) (XOR inside aligned groups of 8).
// V tile: key t, chunk c at slot VC*t + (c ^ v_swz(t)).  Both keep the 16-lane passes of
// ds_read_b128 (score operand) and the 32-lane passes of ds_read_b64_tr_b16 (value
// operand) on distinct banks.
__device__ __forceinline__ int k_swz(int t) { return (t >> 1) & 7; }
__device__ __forceinline__ int v_swz(int t) { return 2 * (t & 7); }

struct PrefillArgs {
  const bf16_t* q;
  const bf16_t* k;
  const bf16_t* v;
  bf16_t* o;
  int T, H;
  float scale_log2;
  int n_qtiles;
};

// Copies of key tile kt: NW waves share K_SLOTS + V_SLOTS 16-byte slots.  Keys past T
// repeat the last key (their scores are masked).  Offsets are taken from the tile's first
// row of head h, so they stay far below 4 GB.
template <int NW>
__device__ __forceinline__ void issue_kv_copy(const PrefillArgs& P, int h, int kt, uint4* __restrict__ kb,
                                              uint4* __restrict__ vb, int w, int lane) {
  int l = lane;
  asm volatile("" : "+v"(l));
  constexpr int KI = K_SLOTS / 64 / NW, VI = V_SLOTS / 64 / NW;
  const int k0 = kt * KT, t_max = P.T - 1 - k0;
  const bf16_t* kbase = P.k + ((int64_t)k0 * P.H + h) * DQK;
  const bf16_t* vbase = P.v + ((int64_t)k0 * P.H + h) * DV;
#pragma unroll
  for (int i = 0; i < KI; ++i) {
    const int p = 64 * (KI * w + i) + l;
    const int t = p / KC, c = (p - t * KC) ^ k_swz(t);
    const int tt = min(t, t_max);
    dma16_buf(kbase, 0x7FFFFFF0u, (uint32_t)((tt * P.H * DQK + 8 * c) * 2), kb + 64 * (KI * w + i));
  }
#pragma unroll
  for (int i = 0; i < VI; ++i) {
    const int p = 64 * (VI * w + i) + l;
    const int t = p / VC, c = (p - t * VC) ^ v_swz(t);
    const int tt = min(t, t_max);
    dma16_buf(vbase, 0x7FFFFFF0u, (uint32_t)((tt * P.H * DV + 8 * c) * 2), vb + 64 * (VI * w + i));
  }
}

template <int NW>
__device__ __forceinline__ void prefill_tile(const PrefillArgs& P, int h, int kt, bool copy, int kt_pf, bool compute,
                                             int qw0, const uint4* __restrict__ kb, const uint4* __restrict__ vb,
                                             uint4* __restrict__ kn, uint4* __restrict__ vn,
                                             const bf16x8 (&qf)[2][DQK / 32], f32x4 (&o)[DV / 16][2],
                                             float (&m_run)[2], float (&l_run)[2], const int (&kbase)[2],
                                             const int (&vbase)[4], int w, int lane) {
  const int g = lane >> 4, j = lane & 15;
  if (copy) issue_kv_copy<NW>(P, h, kt_pf, kn, vn, w, lane);
  const int k0 = kt * KT;
  if (compute && k0 <= qw0 + 31) {  // this wave has queries that see keys of the tile
    // ---- S^T[key][query]
    f32x4 s[4][2];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) s[mt][0] = s[mt][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < DQK / 32; ++ks) {
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        // slot KC*(16*mt + j) + ((4*ks + g) ^ k_swz(j)), lane part in kbase[ks & 1]
        const bf16x8 a = as_bf16x8(*(const uint4*)((const char*)kb + kbase[ks & 1] + (KC * 16 * mt + 8 * (ks >> 1)) * 16));
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) s[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[nt][ks], s[mt][nt], 0, 0, 0);
      }
    }
    // ---- online softmax per query (lane's query: qw0 + 16*nt + j).  Every query sees key 0 in
    // tile 0 (computed by every wave), so the running max is finite from the first tile on.
    const bool diag = k0 + KT - 1 > qw0;
    bf16x8 pb[2][2];  // [nt][kk]
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      float x[4][4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) x[mt][i] = s[mt][nt][i] * P.scale_log2;
      if (diag) {  // causal mask inside the diagonal tiles only
        const int qi = qw0 + 16 * nt + j;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (k0 + 16 * mt + 4 * g + i > qi) x[mt][i] = -INFINITY;
      }
      float mx = x[0][0];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) mx = fmaxf(mx, x[mt][i]);
      mx = xmax16_32(mx);
      const float m_new = (m_run[nt] == -INFINITY || mx > m_run[nt] + kRescaleThreshold) ? mx : m_run[nt];
      const float corr = m_run[nt] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run[nt] - m_new);
      float sum = 0.f;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        float p[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          p[i] = __builtin_amdgcn_exp2f(x[2 * kk][i] - m_new);
          p[4 + i] = __builtin_amdgcn_exp2f(x[2 * kk + 1][i] - m_new);
          sum += p[i] + p[4 + i];
        }
        pb[nt][kk] = as_bf16x8(make_uint4(pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]), pack_bf16x2(p[4], p[5]), pack_bf16x2(p[6], p[7])));
      }
      sum = xsum16_32(sum);
      l_run[nt] = l_run[nt] * corr + sum;
      m_run[nt] = m_new;
      if (__any(corr != 1.f)) {
#pragma unroll
        for (int mt = 0; mt < DV / 16; ++mt) o[mt][nt] *= corr;
      }
    }
    // ---- O^T[d][query] += V^T P^T
    const char* vbb = (const char*)vb;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
      for (int mt = 0; mt < DV / 16; ++mt) {
        // keys 32*kk + {0,16} + 4*g + j/4 (same swizzle), chunk 2*mt + half = (2*mt) ^ half
        const char* pa = vbb + vbase[0] + (VC * 32 * kk) * 16 + ((2 * mt) ^ vbase[1]) * 16;
        const bf16x4 a0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)pa);
        const bf16x4 a1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(pa + VC * 16 * 16));
        const bf16x8 a = __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) o[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pb[nt][kk], o[mt][nt], 0, 0, 0);
      }
    }
  }
}

constexpr int kStages = 3;  // K/V tiles in LDS: the current one and two in flight

template <int NW>
__global__ __launch_bounds__(64 * NW, 1) void prefill_attn_kernel(PrefillArgs P) {
  __shared__ __attribute__((aligned(16))) uint4 kbuf[kStages][K_SLOTS];
  __shared__ __attribute__((aligned(16))) uint4 vbuf[kStages][V_SLOTS];
  constexpr int BQ = 32 * NW;
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, j = lane & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  // block -> (head, query tile): one XCD per group of heads, heaviest query tiles first
  const int bid = blockIdx.x;
  const int per_xcd = (P.H * P.n_qtiles + kXcds - 1) / kXcds;
  const int lin = (bid % kXcds) * per_xcd + bid / kXcds;
  if (lin >= P.H * P.n_qtiles) return;
  const int h = lin / P.n_qtiles;
  const int qt = P.n_qtiles - 1 - (lin - h * P.n_qtiles);
  const int q0 = qt * BQ, qw0 = q0 + 32 * w;
  const int q_last = min(P.T, q0 + BQ) - 1;
  const int n_kt = q_last / KT + 1;

  int kbase[2], vbase[4];
  {
    const int sj = k_swz(j);
#pragma unroll
    for (int e = 0; e < 2; ++e) kbase[e] = (KC * j + ((4 * e + g) ^ sj)) * 16;
    const int tA = 4 * g + (j >> 2), half = (j >> 1) & 1;
    vbase[0] = VC * tA * 16 + (j & 1) * 8;   // row part
    vbase[1] = half ^ v_swz(tA);            // chunk XOR
    vbase[2] = vbase[3] = 0;
  }
  bf16x8 qf[2][DQK / 32];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int qi = min(qw0 + 16 * nt + j, P.T - 1);
    const bf16_t* qrow = P.q + ((int64_t)qi * P.H + h) * DQK + 8 * g;
#pragma unroll
    for (int ks = 0; ks < DQK / 32; ++ks) qf[nt][ks] = as_bf16x8(*(const uint4*)(qrow + 32 * ks));
  }
  f32x4 o[DV / 16][2];
#pragma unroll
  for (int mt = 0; mt < DV / 16; ++mt) o[mt][0] = o[mt][1] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run[2] = {-INFINITY, -INFINITY}, l_run[2] = {0.f, 0.f};
  // the query fragments are complete before the loop, so no read in it waits for the copies
  __builtin_amdgcn_s_waitcnt(0);
  constexpr int kCopies = (K_SLOTS + V_SLOTS) / 64 / NW;  // per wave per tile
  typedef __attribute__((address_space(3))) uint4 lds_uint4;
  // steps kt < 0 only put the first kStages - 1 tiles in flight
  for (int kt = -(kStages - 1); kt < n_kt; ++kt) {
    if (kt >= 0) {
      // copies issued after tile kt's: those of the next min(kStages - 2, ...) tiles
      if (kt + 1 < n_kt) __builtin_amdgcn_s_waitcnt(0x0F70 | kCopies);
      else __builtin_amdgcn_s_waitcnt(0x0F70);
      lds_barrier();
    }
    const int kt_pf = kt + kStages - 1;
    const int b_pf = (kt_pf + kStages) % kStages, b_cur = kt < 0 ? 0 : kt % kStages;
    // opaque copies of the buffer pointers keep the restrict scopes of prefill_tile's parameters
    lds_uint4 *kc = (lds_uint4*)kbuf[b_cur], *vc = (lds_uint4*)vbuf[b_cur];
    lds_uint4 *kn = (lds_uint4*)kbuf[b_pf], *vn = (lds_uint4*)vbuf[b_pf];
    asm volatile("" : "+s"(kc), "+s"(vc), "+s"(kn), "+s"(vn));
    prefill_tile<NW>(P, h, kt < 0 ? 0 : kt, kt_pf < n_kt, kt_pf, kt >= 0, qw0, (const uint4*)kc, (const uint4*)vc,
                     (uint4*)kn, (uint4*)vn, qf, o, m_run, l_run, kbase, vbase, w, lane);
  }
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int qi = qw0 + 16 * nt + j;
    if (qi >= P.T) continue;
    const float inv = l_run[nt] > 0.f ? 1.f / l_run[nt] : 0.f;
    bf16_t* dst = P.o + ((int64_t)qi * P.H + h) * DV + 4 * g;
#pragma unroll
    for (int mt = 0; mt < DV / 16; ++mt) {
      const f32x4 v = o[mt][nt] * inv;
      *(uint2*)(dst + 16 * mt) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
    }
  }
}

}  // namespace

bool fast_prefill_attn_supported(const Dims& d) { return d.act == 1 && d.dn + d.dr == DQK && d.dv == DV; }

size_t fast_prefill_attn_ws_bytes(const Dims&, int) { return 0; }

hipError_t fast_prefill_attn(const Dims& d, const void* q, const void* k, const void* v, int T, void* o, void*,
                             hipStream_t s) {
  PrefillArgs P;
  P.q = (const bf16_t*)q;
  P.k = (const bf16_t*)k;
  P.v = (const bf16_t*)v;
  P.o = (bf16_t*)o;
  P.T = T;
  P.H = d.H;
  P.scale_log2 = d.scale * 1.4426950408889634f;
  // 256 queries per workgroup when that still gives every CU work, else 128
  const bool big = (int64_t)d.H * ((T + 255) / 256) >= 1024;
  const int BQ = big ? 256 : 128;
  P.n_qtiles = (T + BQ - 1) / BQ;
  const int total = d.H * P.n_qtiles;
  const int grid = (total + kXcds - 1) / kXcds * kXcds;
  if (big) prefill_attn_kernel<8><<<grid, 512, 0, s>>>(P);
  else prefill_attn_kernel<4><<<grid, 256, 0, s>>>(P);
  return hipGetLastError();
}

}  // namespace mla
