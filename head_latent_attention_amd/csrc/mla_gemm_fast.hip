// Projection GEMM / GEMV on CDNA4 matrix cores (gfx950):
//   C[M, N] (fp32) = A[M, K] (bf16, row-major) @ [W0 | W1] (bf16, or E4M3FN bytes with
//   fp32 128x128 block scales), weights in the [in, out] orientation the NKI projection
//   kernels take.  Two weights that read the same activations (the query and kv
//   down-projections) run as one launch: W0 feeds output columns [0, n_split), W1 the
//   rest.
//
// One workgroup (4 waves) owns a BM x 128 output tile and a K range; K advances in
// steps of 64 through double-buffered LDS tiles loaded via registers.  A is read
// with ds_read_b128 (row-contiguous k); W is stored row-major [k][n] and the B
// operand (k-contiguous per lane) comes from the gfx950 transposing read
// ds_read_b64_tr_b16.  fp8 weights are decoded to bf16 while being staged: the
// E4M3FN value times a power-of-two block scale is exact in bf16, so the matrix
// op sees the same numbers the block-scaled weight represents (atlas "Struct
// MlaWeights", fp8 fields: the GEMV reads one byte per weight and dequantises in
// the kernel).  Skinny decode shapes split K over extra workgroups; the result is
// handed on as the split-K partial sums, which the consuming kernel adds in a fixed
// order, so results are bitwise reproducible.
#include "mla_fast.h"

namespace mla {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

constexpr int BK = 64;   // k per LDS stage
constexpr int BN = 128;  // output columns per workgroup

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

// A tile: [BM][64] bf16, 8 chunks of 16 B per row; chunk c of row r at slot 8r + (c ^ ((r >> 1) & 7)).
__device__ __forceinline__ int a_slot(int r, int c) { return 8 * r + (c ^ ((r >> 1) & 7)); }
// W tile: [64][128] bf16, 16 chunks per row; chunk c of row k at slot 16k + (c ^ ws(k)).  The XOR
// patterns keep the 16-lane passes of ds_read_b128 and the 32-lane passes of the transposing
// ds_read_b64_tr_b16 on distinct banks.
__device__ __forceinline__ int w_slot(int k, int c) { return 16 * k + (c ^ (((k & 3) << 1) ^ (((k >> 3) & 1) << 3))); }

template <int BM, int WM, int WN, int WK>
struct Gemm {
  static constexpr int MT = BM / WM / 16;   // 16-row tiles per wave
  static constexpr int NT = BN / WN / 16;   // 16-col tiles per wave
  static constexpr int A_LOADS = BM * 8 / 256;  // 16-byte chunks of A per thread
  static constexpr int W_LOADS = 4;             // bf16 chunks of W per thread (fp8: 2 loads, 4 chunks after decode)
  static constexpr int A_SLOTS = BM * 8, W_SLOTS = BK * 16;
  static_assert(WM * WN == 4, "4 waves");
};

struct EpiArgs {
  int kind;
  bf16_t* y;
  bf16_t* y2;
  const float* cosT;
  const float* sinT;
  int H, dn, dr, dv;
  int kind1 = GemmEpilogue::PARTIALS;  // the large-tile kernels: consumer of the W1 segment's tiles
  int64_t ldy = 0;                     // row stride of y for STORE / QUERY (0: N)
};

// Epilogue of the BM x 128 tile kernels (4 waves; acc[mt][nt][i] is tile row
// wm*(BM/WM) + 16*mt + 4*g + i, column wn*(128/WN) + 16*nt + j).
template <int BM, int WM, int WN>
__device__ __forceinline__ void small_epilogue(const EpiArgs& E, f32x4 (&acc)[BM / WM / 16][BN / WN / 16], float* C,
                                               int64_t ldc, int M, int N, int m0, int n0, int wm, int wn, int lane) {
  using G = Gemm<BM, WM, WN, W_BF16>;
  const int g = lane >> 4, j = lane & 15;
  const int wcol0 = wn * (BN / WN);
  if (E.kind == GemmEpilogue::PARTIALS) {
#pragma unroll
    for (int mt = 0; mt < G::MT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = m0 + wm * (BM / WM) + 16 * mt + 4 * g + i;
        if (m >= M) continue;
#pragma unroll
        for (int nt = 0; nt < G::NT; ++nt) {
          const int n = n0 + wcol0 + 16 * nt + j;
          if (n < N) C[(int64_t)m * ldc + n] = acc[mt][nt][i];
        }
      }
    return;
  }
  // consumers: column n of the lane (j) and its RoPE partner n ^ 1 (lane j ^ 1, same rows)
  const int dqk = E.dn + E.dr, half = E.dr >> 1, dkv = E.dn + E.dv;
#pragma unroll
  for (int nt = 0; nt < G::NT; ++nt) {
    const int n = n0 + wcol0 + 16 * nt + j;
    int h = 0, u = 0;
    if (E.kind == GemmEpilogue::QUERY) { h = n / dqk; u = n - h * dqk; }
    if (E.kind == GemmEpilogue::KV) { h = n / dkv; u = n - h * dkv; }
#pragma unroll
    for (int mt = 0; mt < G::MT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = m0 + wm * (BM / WM) + 16 * mt + 4 * g + i;
        const float x = acc[mt][nt][i];
        const float other = __shfl_xor(x, 1);  // every lane takes part
        if (m >= M || n >= N) continue;
        if (E.kind == GemmEpilogue::STORE) {
          E.y[(int64_t)m * N + n] = f32_to_bf16(x);
        } else if (E.kind == GemmEpilogue::QUERY) {
          float yv = x;
          if (u >= E.dn) {
            const int p = (u - E.dn) >> 1;
            const float c = E.cosT[(int64_t)m * half + p], sn = E.sinT[(int64_t)m * half + p];
            yv = (u - E.dn) & 1 ? other * sn + x * c : x * c - other * sn;
          }
          E.y[(int64_t)m * N + n] = f32_to_bf16(yv);
        } else {
          if (u < E.dn) E.y[((int64_t)m * E.H + h) * dqk + u] = f32_to_bf16(x);
          else E.y2[((int64_t)m * E.H + h) * E.dv + (u - E.dn)] = f32_to_bf16(x);
        }
      }
  }
}

template <int BM, int WM, int WN, int WK>
__global__ __launch_bounds__(256) void gemm_kernel(const bf16_t* __restrict__ A, int64_t lda, WeightView W0,
                                                   WeightView W1, int n_split, float* __restrict__ C, int64_t ldc,
                                                   int M, int N, int K, int k_split, int64_t split_stride,
                                                   EpiArgs E) {
  using G = Gemm<BM, WM, WN, WK>;
  __shared__ __attribute__((aligned(16))) uint4 As[2][G::A_SLOTS];
  __shared__ __attribute__((aligned(16))) uint4 Ws[2][G::W_SLOTS];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, g = lane >> 4, j = lane & 15;
  const int wm = wv / WN, wn = wv % WN;
  const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
  const int kbeg = blockIdx.z * k_split, kend = min(K, kbeg + k_split);
  C += (int64_t)blockIdx.z * split_stride;
  // weight segment of this column tile (n_split is a multiple of BN, so a tile never straddles it)
  const bool seg1 = n0 >= n_split;
  const WeightView W = seg1 ? W1 : W0;
  const int wn0 = seg1 ? n0 - n_split : n0, WN_ = seg1 ? N - n_split : n_split;

  uint4 ra[G::A_LOADS], rw[G::W_LOADS];
  auto load = [&](int k0) {
#pragma unroll
    for (int it = 0; it < G::A_LOADS; ++it) {
      const int e = it * 256 + tid, r = e >> 3, c = e & 7;
      const int m = m0 + r, k = k0 + 8 * c;
      ra[it] = (m < M && k < kend) ? *(const uint4*)(A + (int64_t)m * lda + k) : make_uint4(0, 0, 0, 0);
    }
    if constexpr (WK == W_BF16) {
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        const int e = it * 256 + tid, kr = e >> 4, c = e & 15;
        const int k = k0 + kr, n = wn0 + 8 * c;
        rw[it] = (k < kend && n < WN_) ? *(const uint4*)((const bf16_t*)W.w + (int64_t)k * W.ld + n)
                                     : make_uint4(0, 0, 0, 0);
      }
    } else {
      // 64 x 128 bytes = 512 chunks of 16 B; thread takes 2, each becomes 2 bf16 chunks
#pragma unroll
      for (int it = 0; it < 2; ++it) {
        const int e = it * 256 + tid, kr = e >> 3, c = e & 7;
        const int k = k0 + kr, n = wn0 + 16 * c;
        uint4 raw = make_uint4(0, 0, 0, 0);
        float s = 0.f;
        if (k < kend && n < WN_) {
          raw = *(const uint4*)((const uint8_t*)W.w + (int64_t)k * W.ld + n);
          s = W.scale[(k >> 7) * W.scale_ld + (n >> 7)];
        }
        uint32_t words[4] = {raw.x, raw.y, raw.z, raw.w};
        uint32_t out[8];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)words[q], false);
          const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)words[q], true);
          out[2 * q] = pack_bf16x2(lo[0] * s, lo[1] * s);
          out[2 * q + 1] = pack_bf16x2(hi[0] * s, hi[1] * s);
        }
        rw[2 * it] = make_uint4(out[0], out[1], out[2], out[3]);
        rw[2 * it + 1] = make_uint4(out[4], out[5], out[6], out[7]);
      }
    }
  };
  auto store = [&](uint4* __restrict__ as, uint4* __restrict__ ws) {
#pragma unroll
    for (int it = 0; it < G::A_LOADS; ++it) {
      const int e = it * 256 + tid;
      as[a_slot(e >> 3, e & 7)] = ra[it];
    }
    if constexpr (WK == W_BF16) {
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        const int e = it * 256 + tid;
        ws[w_slot(e >> 4, e & 15)] = rw[it];
      }
    } else {
#pragma unroll
      for (int it = 0; it < 2; ++it) {
        const int e = it * 256 + tid, kr = e >> 3, c = e & 7;
        ws[w_slot(kr, 2 * c)] = rw[2 * it];
        ws[w_slot(kr, 2 * c + 1)] = rw[2 * it + 1];
      }
    }
  };

  f32x4 acc[G::MT][G::NT];
#pragma unroll
  for (int a = 0; a < G::MT; ++a)
#pragma unroll
    for (int b = 0; b < G::NT; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

  // lane parts of the LDS addresses
  const int arow0 = wm * (BM / WM) + j;                  // + 16*mt
  const int wcol0 = wn * (BN / WN);                      // + 16*nt
  if (kbeg < kend) {
    load(kbeg);
    store(As[0], Ws[0]);
  }
  __syncthreads();
  int cur = 0;
  for (int k0 = kbeg; k0 < kend; k0 += BK) {
    const bool next = k0 + BK < kend;
    if (next) load(k0 + BK);
    const uint4* as = As[cur];
    const char* wsb = (const char*)Ws[cur];
#pragma unroll
    for (int ks = 0; ks < BK / 32; ++ks) {
      bf16x8 af[G::MT], bfr[G::NT];
#pragma unroll
      for (int mt = 0; mt < G::MT; ++mt) af[mt] = as_bf16x8(as[a_slot(arow0 + 16 * mt, 4 * ks + g)]);
#pragma unroll
      for (int nt = 0; nt < G::NT; ++nt) {
        const int col = wcol0 + 16 * nt + 4 * (j & 3);
        const int c = col >> 3, byte_in = (col & 7) * 2;
        const int k = 32 * ks + 8 * g + (j >> 2);
        const bf16x4 b0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(wsb + w_slot(k, c) * 16 + byte_in));
        const bf16x4 b1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(wsb + w_slot(k + 4, c) * 16 + byte_in));
        bfr[nt] = __builtin_shufflevector(b0, b1, 0, 1, 2, 3, 4, 5, 6, 7);
      }
#pragma unroll
      for (int mt = 0; mt < G::MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < G::NT; ++nt)
          acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[mt], bfr[nt], acc[mt][nt], 0, 0, 0);
    }
    if (next) store(As[cur ^ 1], Ws[cur ^ 1]);
    __syncthreads();
    cur ^= 1;
  }
  small_epilogue<BM, WM, WN>(E, acc, C, ldc, M, N, m0, n0, wm, wn, lane);
}

// ---------------------------------------------------------------------------------------------
// Decode variant (M <= 64, bf16 weights): the 64 x 128 tile and 4-wave layout of gemm_kernel, but
// the K steps are copied global->LDS by buffer_load ... lds three stages deep (two steps in
// flight while one is multiplied), so that the weight stream of a workgroup is not one load
// latency per step.  Each K range must be a whole number of 64-wide steps.
constexpr int kDecStages = 3;
constexpr int kDecCopies = 6;  // per wave per step: 2 activation + 4 weight copies of 1 KB

struct DecArgs {
  const bf16_t* A;
  int64_t lda;
  WeightView W0, W1;
  int n_split;
  float* C;
  int64_t ldc;
  int M, N, K;
  int k_split;
  int64_t split_stride;
};

// Copies of K step k0 into one stage (A: [64][8 chunks], W: [64][16 chunks], swizzled as
// a_slot / w_slot, so each lane fetches the global chunk that belongs at its LDS slot).  Rows
// past M and columns past the segment are clamped to valid memory; they only feed outputs
// that are not stored.
__device__ __forceinline__ void dec_issue(const DecArgs& G, const WeightView& W, int wn0, int wn_end, int k0,
                                          uint4* __restrict__ as, uint4* __restrict__ ws, int w, int lane) {
  int l = lane;
  asm volatile("" : "+v"(l));
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int e = 64 * (2 * w + i) + l, r = e >> 3, c = (e & 7) ^ ((r >> 1) & 7);
    const int m = min(r, G.M - 1);
    dma16_buf(G.A + k0, 0x7FFFFFF0u, (uint32_t)((m * G.lda + 8 * c) * 2), as + 64 * (2 * w + i));
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = 64 * (4 * w + i) + l, kr = e >> 4, c = (e & 15) ^ (((kr & 3) << 1) ^ (((kr >> 3) & 1) << 3));
    const int n = min(wn0 + 8 * c, wn_end - 8);
    dma16_buf((const bf16_t*)W.w + (int64_t)k0 * W.ld, 0x7FFFFFF0u, (uint32_t)((kr * W.ld + n) * 2),
              ws + 64 * (4 * w + i));
  }
}

// One step: copies of a later step into (as_nx, ws_nx), then the matrix ops of the step in
// (as, ws).  All LDS accesses of the loop are made here through restrict-qualified pointers,
// so the operand reads never wait for the copies in flight.
__device__ __forceinline__ void dec_step(const DecArgs& G, const WeightView& W, int wn0, int wn_end, bool copy, int k_pf,
                                         bool compute, const uint4* __restrict__ as, const uint4* __restrict__ ws,
                                         uint4* __restrict__ as_nx, uint4* __restrict__ ws_nx, f32x4 (&acc)[4][2],
                                         int w, int lane) {
  if (copy) dec_issue(G, W, wn0, wn_end, k_pf, as_nx, ws_nx, w, lane);
  if (!compute) return;
  const int g = lane >> 4, j = lane & 15;
  const char* wsb = (const char*)ws;
#pragma unroll
  for (int ks = 0; ks < BK / 32; ++ks) {
    bf16x8 af[4], bfr[2];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) af[mt] = as_bf16x8(as[a_slot(16 * mt + j, 4 * ks + g)]);
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const int col = 32 * w + 16 * nt + 4 * (j & 3);
      const int c = col >> 3, byte_in = (col & 7) * 2;
      const int k = 32 * ks + 8 * g + (j >> 2);
      const bf16x4 b0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(wsb + w_slot(k, c) * 16 + byte_in));
      const bf16x4 b1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(wsb + w_slot(k + 4, c) * 16 + byte_in));
      bfr[nt] = __builtin_shufflevector(b0, b1, 0, 1, 2, 3, 4, 5, 6, 7);
    }
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
        acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[mt], bfr[nt], acc[mt][nt], 0, 0, 0);
  }
}

// bf16 epilogue of the 64 x 128 decode tile (STORE, or QUERY with RoPE on the query's rope
// columns): the tile is staged in LDS (`st`, 16 KB of idle stage buffers; 256-byte rows of
// 16-byte chunks, chunk c of row r at slot 16r + (c ^ (r & 15))) so that every global store is
// a whole 16-byte chunk of 8 columns.  acc[mt][nt][i] is tile row 16mt + 4g + i, column
// 32w + 16nt + j; the cos/sin of a lane's 16 rows are all loaded before the first use, and the
// pair partner of a rope column sits in lane j ^ 1.
__device__ __forceinline__ void dec_store_epilogue(const EpiArgs& E, f32x4 (&acc)[4][2], bf16_t* st, int M, int N,
                                                   int n0, int w, int lane) {
  const int tid = threadIdx.x, g = lane >> 4, j = lane & 15;
  const int dqk = E.dn + E.dr, half = E.dr >> 1;
  auto chunk_of = [](int r, int c) { return 16 * r + (c ^ (r & 15)); };
  const bool query = E.kind == GemmEpilogue::QUERY;
  lds_barrier();  // every wave is done with the stage buffers
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int c = 32 * w + 16 * nt + j;
    const int u = (n0 + c) % dqk;
    const bool rope = query && u >= E.dn, odd = (u - E.dn) & 1;
    const int p = (u - E.dn) >> 1;
    float cs[4][4], sn[4][4];
    if (rope) {
      const uint32_t tbytes = (uint32_t)min((int64_t)M * half * 4, (int64_t)0x7FFFFFF0);
      const __amdgpu_buffer_rsrc_t rc = __builtin_amdgcn_make_buffer_rsrc((void*)E.cosT, 0, (int)tbytes, 0x00020000);
      const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void*)E.sinT, 0, (int)tbytes, 0x00020000);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t off = (uint32_t)((min(16 * mt + 4 * g + i, M - 1) * half + p) * 4);
          cs[mt][i] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rc, off, 0, 0));
          sn[mt][i] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, 0));
        }
    }
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      float y[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        y[i] = acc[mt][nt][i];
        if (query) {
          const float other = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(y[i]), 0xB1, 0xF, 0xF, true));
          if (rope) y[i] = odd ? other * sn[mt][i] + y[i] * cs[mt][i] : y[i] * cs[mt][i] - other * sn[mt][i];
        }
      }
      // lanes j and j ^ 1 hold columns c and c ^ 1 of the same 4 rows: swapping one value per row
      // pair gives the even lane both columns of row i, the odd lane both of row i + 1
      const int c0 = c & ~1;
#pragma unroll
      for (int i = 0; i < 4; i += 2) {
        const float send = (j & 1) ? y[i] : y[i + 1];
        const float recv = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(send), 0xB1, 0xF, 0xF, true));
        const int r = 16 * mt + 4 * g + i + (j & 1);
        const uint32_t pk = (j & 1) ? pack_bf16x2(recv, y[i + 1]) : pack_bf16x2(y[i], recv);
        *(uint32_t*)&st[chunk_of(r, c0 >> 3) * 8 + (c0 & 7)] = pk;
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's part of the tile is in LDS
  lds_barrier();
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int e = it * 256 + tid, r = e >> 4, c8 = e & 15;
    const int n = n0 + 8 * c8;
    if (r < M && n < N) *(uint4*)&E.y[(int64_t)r * N + n] = *(const uint4*)&st[chunk_of(r, c8) * 8];
  }
}

__global__ __launch_bounds__(256) void gemm_dec_kernel(DecArgs G, EpiArgs E) {
  __shared__ __attribute__((aligned(16))) uint4 As[kDecStages][64 * 8];
  __shared__ __attribute__((aligned(16))) uint4 Ws[kDecStages][BK * 16];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n0 = blockIdx.x * BN;
  const bool seg1 = n0 >= G.n_split;
  const WeightView W = seg1 ? G.W1 : G.W0;
  const int wn0 = seg1 ? n0 - G.n_split : n0, wn_end = seg1 ? G.N - G.n_split : G.n_split;
  const int kbeg = blockIdx.z * G.k_split;
  const int nsteps = (min(G.K, kbeg + G.k_split) - kbeg) / BK;
  f32x4 acc[4][2];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) acc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int s = -(kDecStages - 1); s < nsteps; ++s) {
    if (s >= 0) {
      // copies issued after step s's: those of the next step, if any
      if (s + 1 < nsteps) __builtin_amdgcn_s_waitcnt(0x0F70 | kDecCopies);
      else __builtin_amdgcn_s_waitcnt(0x0F70);
      lds_barrier();
    }
    const int s_pf = s + kDecStages - 1;
    const int b_pf = (s_pf + kDecStages) % kDecStages, b_cur = s < 0 ? 0 : s % kDecStages;
    // opaque copies of the stage pointers keep the restrict scopes of dec_step's parameters
    typedef __attribute__((address_space(3))) uint4 lds_uint4;
    lds_uint4 *a_cur = (lds_uint4*)As[b_cur], *w_cur = (lds_uint4*)Ws[b_cur];
    lds_uint4 *a_nx = (lds_uint4*)As[b_pf], *w_nx = (lds_uint4*)Ws[b_pf];
    asm volatile("" : "+s"(a_cur), "+s"(w_cur), "+s"(a_nx), "+s"(w_nx));
    dec_step(G, W, wn0, wn_end, s_pf < nsteps, kbeg + s_pf * BK, s >= 0, (const uint4*)a_cur, (const uint4*)w_cur,
             (uint4*)a_nx, (uint4*)w_nx, acc, w, lane);
  }
  if (E.kind == GemmEpilogue::PARTIALS) {
    // the fp32 tile through the idle stage buffers (rows of 128 floats padded to 132), so that
    // every store is 16 bytes and every wave writes two whole 512-byte rows at a time
    lds_barrier();  // every wave is done with the last step's operands
    float* st = (float*)&Ws[0][0];
    static_assert(sizeof(Ws) >= 64 * 132 * 4, "the weight stages hold the tile");
    const int g = lane >> 4, j = lane & 15;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i) st[(16 * mt + 4 * g + i) * 132 + 32 * w + 16 * nt + j] = acc[mt][nt][i];
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    lds_barrier();
    float* C = G.C + (int64_t)blockIdx.z * G.split_stride;
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      const int e = it * 256 + tid, r = e >> 5, c4 = e & 31;
      const int n = n0 + 4 * c4;
      if (r < G.M && n < G.N) *(float4*)&C[(int64_t)r * G.ldc + n] = *(const float4*)&st[r * 132 + 4 * c4];
    }
    return;
  }
  if (E.kind == GemmEpilogue::STORE || E.kind == GemmEpilogue::QUERY) {
    dec_store_epilogue(E, acc, (bf16_t*)&Ws[0][0], G.M, G.N, n0, w, lane);
    return;
  }
  small_epilogue<64, 1, 4>(E, acc, G.C + (int64_t)blockIdx.z * G.split_stride, G.ldc, G.M, G.N, 0, n0, 0, w, lane);
}

bool dec_ok(const Dims& d, int M, int N, int K, int k_split, int n_split, int64_t lda, const float* C, int64_t ldc,
            int64_t split_stride) {
  // every K range a whole number of steps; byte offsets of a step fit 32 bits
  return d.wk == W_BF16 && M <= 64 && K % BK == 0 && k_split % BK == 0 && N % 8 == 0 && ldc % 4 == 0 &&
         split_stride % 4 == 0 && ((uintptr_t)C & 15) == 0 &&
         (n_split >= N || (n_split % BN == 0 && (N - n_split) % 8 == 0)) && (int64_t)64 * lda * 2 < 0x7FFFFFF0LL;
}

// ---------------------------------------------------------------------------------------------
// Large-M variant (prefill): a 256 x 256 output tile per workgroup of 8 waves (2 x 4, each
// 128 x 64), K steps of 32 copied global->LDS by buffer_load ... lds four stages deep.  Each
// LDS operand read feeds 4 (A) or 8 (B) matrix ops instead of 2 and 2 in gemm_kernel.  K and
// the column split must be multiples of 32 and 256.
constexpr int kBigM = 256, kBigN = 256, kBigK = 32, kBigStages = 4;
constexpr int kBigCopies = 4;  // per wave per stage: 2 activation + 2 weight copies of 1 KB

// A stage: [256 rows][4 chunks of 16 B]; chunk c of row r at slot 4r + (c ^ a4_swz(r)), which
// keeps every 16-lane pass of the operand reads on distinct banks.
__device__ __forceinline__ int a4_swz(int r) { return ((r >> 2) & 1) | ((((r >> 2) ^ (r >> 3)) & 1) << 1); }

struct BigArgs {
  const bf16_t* A;
  int64_t lda;
  WeightView W0, W1;
  int n_split;
  float* C;
  int64_t ldc;
  int M, N, K;
  int k_split;           // K range per workgroup along grid z (partial sums)
  int64_t split_stride;  // elements between the partial sums of consecutive ranges
};

// A lane's byte offsets of its copies within a K step (two activation, two weight), the same
// for every step of a tile.  Rows past M and columns past the segment are clamped to valid
// memory; they only feed outputs that are not stored.
struct BigCopyPlan {
  uint32_t off[4];
};

__device__ __forceinline__ BigCopyPlan big_offsets(const BigArgs& G, const WeightView& W, int m0, int wn0, int wn_end,
                                                   int w, int lane) {
  BigCopyPlan cp;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int e = 64 * (2 * w + i) + lane, r = e >> 2, c = (e & 3) ^ a4_swz(r);
    const int m = min(m0 + r, G.M - 1);
    cp.off[i] = (uint32_t)((m * G.lda + 8 * c) * 2);
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int blk = 2 * w + i, hb = blk >> 3, e = 64 * (blk & 7) + lane;  // half hb: columns [128hb, 128hb + 128)
    const int kr = e >> 4, c = (e & 15) ^ (((kr & 3) << 1) ^ (((kr >> 3) & 1) << 3));
    const int n = min(wn0 + 128 * hb + 8 * c, wn_end - 8);
    cp.off[2 + i] = (uint32_t)((kr * W.ld + n) * 2);
  }
  return cp;
}

// Copies of K step k0 into one stage.
__device__ __forceinline__ void big_issue(const BigArgs& G, const WeightView& W, const BigCopyPlan& cp, int k0,
                                          uint4* __restrict__ as, uint4* __restrict__ ws, int w) {
#pragma unroll
  for (int i = 0; i < 2; ++i) dma16_buf(G.A + k0, 0x7FFFFFF0u, cp.off[i], as + 64 * (2 * w + i));
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int blk = 2 * w + i, hb = blk >> 3;
    dma16_buf((const bf16_t*)W.w + (int64_t)k0 * W.ld, 0x7FFFFFF0u, cp.off[2 + i], ws + 512 * hb + 64 * (blk & 7));
  }
}

// Operand reads of one stage: A rows 128*wm + 16*mt + j (8 chunks of K), and B columns
// 64*(wn & 1) + 16*nt + .. of the wave's half through the transposing read.
__device__ __forceinline__ bf16x8 big_a(const uint4* __restrict__ as, int mt, int w, int lane) {
  const int r = 128 * (w >> 2) + 16 * mt + (lane & 15);
  return as_bf16x8(as[4 * r + ((lane >> 4) ^ a4_swz(r))]);
}

__device__ __forceinline__ bf16x8 big_b(const uint4* __restrict__ ws, int nt, int w, int lane) {
  const int g = lane >> 4, j = lane & 15, wn = w & 3;
  const char* wsb = (const char*)(ws + 512 * (wn >> 1));
  const int col = 64 * (wn & 1) + 16 * nt + 4 * (j & 3);
  const int c = col >> 3, byte_in = (col & 7) * 2;
  const int k = 8 * g + (j >> 2);
  const bf16x4 b0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(wsb + w_slot(k, c) * 16 + byte_in));
  const bf16x4 b1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(wsb + w_slot(k + 4, c) * 16 + byte_in));
  return __builtin_shufflevector(b0, b1, 0, 1, 2, 3, 4, 5, 6, 7);
}

// One K step: this step's share of the copies into the free stage `as_nx/ws_nx`, then the
// matrix ops of the current stage, whose operands af/bf were read during the previous step.
// The ops run column block by column block (nt outer), so that each operand register is dead
// right after its last op: the B operand of block nt after the block, the A operand of row
// block mt after the last block's op mt.  The operand of the next stage `as1/ws1` is read into
// that register at once, so that every read of the next step is in flight (most of them long
// done) when the barrier in front of it releases, and no wave waits for LDS after a barrier.
// The next stage is complete for this whole step (its copies were waited for, and made visible
// by the barrier, at the top of the step); in the last step the reads return unused values.
// `pre` alone (no compute) reads all operands of the next stage: the first step's.  Every LDS
// access of a step is issued here, through restrict pointers.
__device__ __forceinline__ void big_step(const BigArgs& G, const WeightView& W, const BigCopyPlan& cp, bool copy,
                                         int k_pf, bool compute, bool pre, const uint4* __restrict__ as1,
                                         const uint4* __restrict__ ws1, uint4* __restrict__ as_nx,
                                         uint4* __restrict__ ws_nx, f32x4 (&acc)[8][4], bf16x8 (&af)[8],
                                         bf16x8 (&bf)[4], int w, int lane) {
  if (copy) big_issue(G, W, cp, k_pf, as_nx, ws_nx, w);
  if (compute) {
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      // the B reads after blocks 0 and 1 are long done; retiring them keeps at most 12 LDS reads
      // in flight at the loop's back edge, so that the compiler's count of them stays exact and
      // the next step's first op waits for its own operands only (lgkmcnt(2))
      if (nt == 3) __builtin_amdgcn_s_waitcnt(0xC27F);
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) {
        acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[mt], bf[nt], acc[mt][nt], 0, 0, 0);
        if (nt == 3) af[mt] = big_a(as1, mt, w, lane);
      }
      bf[nt] = big_b(ws1, nt, w, lane);
      __builtin_amdgcn_sched_barrier(0);
    }
  } else if (pre) {
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) bf[nt] = big_b(ws1, nt, w, lane);
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) af[mt] = big_a(as1, mt, w, lane);
    // these 16 reads are more than the LDS counter tracks in order: completing them here keeps
    // the loop's wait model exact
    __builtin_amdgcn_s_waitcnt(0xC07F);
  }
}

// Epilogue of the large-tile kernels: a TM x TN tile (256 x 256 with 8 waves of 128 x 64, or
// 128 x 128 with 4 waves of 64 x 64; acc[mt][nt][i] is tile row (TM/2)*wm + 4*g + 16*mt + i,
// column 64*wn + 16*nt + j).  PARTIALS stores fp32 sums; the bf16 consumers stage the tile in
// LDS (row-major, TN*2-byte rows, 16-byte chunks XOR-swizzled by row; `st` is TM*TN*2 bytes of
// stage buffers no wave reads any more) so that global stores are whole 16-byte chunks of 8
// consecutive columns; the query's RoPE is applied on the way (the partner column of a pair
// sits in lane j ^ 1).
template <int TM, int TN>
__device__ __forceinline__ void big_epilogue(const EpiArgs& E, int kind, f32x4 (&acc)[TM / 32][4], bf16_t* st, int M,
                                             int N, float* C, int64_t ldc, int64_t split_off, int m0, int n0, int w,
                                             int lane) {
  constexpr int NWN = TN / 64, MT = TM / 32, CH = TN / 8;  // waves along N, row tiles, chunks per row
  const int tid = threadIdx.x, g = lane >> 4, j = lane & 15, wm = w / NWN, wn = w % NWN;
  const int dqk = E.dn + E.dr, half = E.dr >> 1, dkv = E.dn + E.dv;
  const int mb = (TM / 2) * wm + 4 * g;  // tile row of acc[mt][.][i]: mb + 16 mt + i
  if (kind == GemmEpilogue::PARTIALS) {
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const int n = n0 + 64 * wn + 16 * nt + j;
      if (n >= N) continue;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int m = m0 + mb + 16 * mt + i;
          if (m < M) C[split_off + (int64_t)m * ldc + n] = acc[mt][nt][i];
        }
    }
    return;
  }
  lds_barrier();  // every wave is done with the stage buffers
  auto chunk_of = [](int r, int c) { return CH * r + (c ^ (r & (CH - 1))); };  // 16-byte chunk slot
  const bool query = kind == GemmEpilogue::QUERY;
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    const int c = 64 * wn + 16 * nt + j;
    const int u = (n0 + c) % dqk;
    const bool rope = query && u >= E.dn, odd = (u - E.dn) & 1;
    const int p = (u - E.dn) >> 1;
    // cos/sin of this lane's pair for 16 rows at a time, all in flight before the first use
    // (the barriers keep the next batch's loads from being hoisted above this one's uses)
    const uint32_t tbytes = (uint32_t)min((int64_t)M * half * 4, (int64_t)0x7FFFFFF0);
#pragma unroll
    for (int hm = 0; hm < MT / 4; ++hm) {
      __builtin_amdgcn_sched_barrier(0);
      float cs[4][4], sn[4][4];
      if (rope) {
        const __amdgpu_buffer_rsrc_t rc = __builtin_amdgcn_make_buffer_rsrc((void*)E.cosT, 0, (int)tbytes, 0x00020000);
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void*)E.sinT, 0, (int)tbytes, 0x00020000);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const uint32_t off = (uint32_t)((min(m0 + mb + 16 * (4 * hm + mt) + i, M - 1) * half + p) * 4);
            cs[mt][i] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rc, off, 0, 0));
            sn[mt][i] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, 0));
          }
      }
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        float y[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          y[i] = acc[4 * hm + mt][nt][i];
          if (query) {
            // the pair partner's value from lane j ^ 1 (DPP quad permutation [1, 0, 3, 2])
            const float other = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(y[i]), 0xB1, 0xF, 0xF, true));
            if (rope) y[i] = odd ? other * sn[mt][i] + y[i] * cs[mt][i] : y[i] * cs[mt][i] - other * sn[mt][i];
          }
        }
        // lanes j and j ^ 1 hold columns c and c ^ 1 of the same 4 rows: swapping one value per
        // row pair gives the even lane both columns of row i, the odd lane both of row i + 1,
        // stored as one 4-byte write each
        const int c0 = c & ~1;
#pragma unroll
        for (int i = 0; i < 4; i += 2) {
          const float send = (j & 1) ? y[i] : y[i + 1];
          const float recv = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(send), 0xB1, 0xF, 0xF, true));
          const int r = mb + 16 * (4 * hm + mt) + i + (j & 1);
          const uint32_t pk = (j & 1) ? pack_bf16x2(recv, y[i + 1]) : pack_bf16x2(y[i], recv);
          *(uint32_t*)&st[chunk_of(r, c0 >> 3) * 8 + (c0 & 7)] = pk;
        }
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's part of the tile is in LDS
  lds_barrier();
  for (int e = tid; e < TM * TN / 8; e += 2 * TN) {  // 2 * TN threads
    const int r = e / CH, c8 = e % CH;
    const int m = m0 + r, n = n0 + 8 * c8;
    if (m >= M || n >= N) continue;
    const uint4 v = *(const uint4*)&st[chunk_of(r, c8) * 8];
    if (kind == GemmEpilogue::KV) {
      const int h = n / dkv, u = n - h * dkv;
      bf16_t* dst = u < E.dn ? E.y + ((int64_t)m * E.H + h) * dqk + u : E.y2 + ((int64_t)m * E.H + h) * E.dv + (u - E.dn);
      *(uint4*)dst = v;
    } else {
      *(uint4*)&E.y[(int64_t)m * (E.ldy > 0 ? E.ldy : N) + n] = v;
    }
  }
}

__global__ __launch_bounds__(512, 1) void gemm_big_kernel(BigArgs G, EpiArgs E) {
  __shared__ __attribute__((aligned(16))) uint4 As[kBigStages][kBigM * 4];
  __shared__ __attribute__((aligned(16))) uint4 Ws[kBigStages][2 * kBigK * 16];
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, j = lane & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = w >> 2, wn = w & 3;
  // column tiles fastest; grid x = column tiles, y = row tiles
  const int n0 = blockIdx.x * kBigN, m0 = blockIdx.y * kBigM;
  const bool seg1 = n0 >= G.n_split;
  const WeightView W = seg1 ? G.W1 : G.W0;
  const int wn0 = seg1 ? n0 - G.n_split : n0, wn_end = seg1 ? G.N - G.n_split : G.n_split;
  const int kbeg = blockIdx.z * G.k_split;
  const int nsteps = (min(G.K, kbeg + G.k_split) - kbeg) / kBigK;
  const BigCopyPlan cp = big_offsets(G, W, m0, wn0, wn_end, w, lane);
  f32x4 acc[8][4];
#pragma unroll
  for (int mt = 0; mt < 8; ++mt)
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) acc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  bf16x8 af[8], bf[4];
#pragma unroll
  for (int i = 0; i < 8; ++i) af[i] = as_bf16x8(make_uint4(0u, 0u, 0u, 0u));
#pragma unroll
  for (int i = 0; i < 4; ++i) bf[i] = as_bf16x8(make_uint4(0u, 0u, 0u, 0u));
  // iteration s: copies of step s+3, matrix ops of step s (s >= 0), operands of step s+1
  for (int s = -(kBigStages - 1); s < nsteps; ++s) {
    if (s >= -1) {
      // steps s and s+1 in LDS: the copies issued after step s+1's are those of step s+2
      if (s + 2 < nsteps) __builtin_amdgcn_s_waitcnt(0x0F70 | kBigCopies);
      else __builtin_amdgcn_s_waitcnt(0x0F70);
      lds_barrier();
    }
    const int s_pf = s + kBigStages - 1;
    const int b_pf = (s_pf + kBigStages) % kBigStages;
    const int b_1 = (s + 1 + kBigStages) % kBigStages;
    // opaque copies of the stage pointers: accesses through them keep the restrict scopes of
    // big_step's parameters (pointers the compiler can trace to the __shared__ arrays lose them,
    // and every operand read would then wait for the copies in flight)
    typedef __attribute__((address_space(3))) uint4 lds_uint4;
    lds_uint4 *a_1 = (lds_uint4*)As[b_1], *w_1 = (lds_uint4*)Ws[b_1];
    lds_uint4 *a_nx = (lds_uint4*)As[b_pf], *w_nx = (lds_uint4*)Ws[b_pf];
    asm volatile("" : "+s"(a_1), "+s"(w_1), "+s"(a_nx), "+s"(w_nx));
    big_step(G, W, cp, s_pf < nsteps, kbeg + s_pf * kBigK, s >= 0, s == -1, (const uint4*)a_1, (const uint4*)w_1,
             (uint4*)a_nx, (uint4*)w_nx, acc, af, bf, w, lane);
  }
  big_epilogue<256, 256>(E, seg1 ? E.kind1 : E.kind, acc, (bf16_t*)&As[0][0], G.M, G.N, G.C, G.ldc,
               (int64_t)blockIdx.z * G.split_stride, m0, n0, w, lane);
}

// ---------------------------------------------------------------------------------------------
// Mid-M projection with fp8 weights (64 < M <= 1024, bf16 activations; the decode step of a
// large batch): the 256 x 256 tile, 8-wave layout, activation stream and epilogue of
// gemm_big_kernel, with the weights kept at one byte per element all the way into LDS.  Each K
// step of 32 copies [32 k][256 n] E4M3 bytes (8 KB, one 16-byte copy per lane) by
// buffer_load ... lds, four stages deep; a wave gets a B operand (8 k of one column per lane)
// from one transposing byte read ds_read_b64_tr_b8 and decodes it in registers: E4M3 -> fp32,
// times the 128 x 128 block scale, -> bf16 (exact for power-of-two block scales, the same
// numbers gemm_kernel's staging produces).  The block scales of the workgroup's K range are
// staged in LDS once, before the first copy.
#ifndef MLA_W8_MIN_KSPLIT
#define MLA_W8_MIN_KSPLIT 512
#endif
constexpr int kW8MinKSplit = MLA_W8_MIN_KSPLIT;  // least K range of one split-K part
#ifndef MLA_W8_STAGES
#define MLA_W8_STAGES 4
#endif
constexpr int kW8Stages = MLA_W8_STAGES;  // K steps in LDS (four and five measured the same;
                                         // six spill registers)
constexpr int kW8Copies = 3;         // per wave per stage: 2 activation + 1 weight copy of 1 KB
constexpr int kW8MaxKBlocks = 128;   // 128-row scale blocks of one workgroup's K range
constexpr int kW8StageA = kBigM * 4, kW8StageW = kBigK * 16;  // 16-byte chunks per stage
// the stages, or the epilogue's 128 KB bf16 tile where that is larger (same array)
constexpr int kW8Smem = kW8Stages * (kW8StageA + kW8StageW) > 8192 ? kW8Stages * (kW8StageA + kW8StageW) : 8192;
static_assert(kW8Stages >= 4 && kW8Smem <= 9216, "stages and the scale table must fit in 160 KB of LDS");

typedef int i32x2w __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i32x2w lds_i32x2w;

// W stage [32 k][16 chunks of 16 columns]: chunk c of row k at slot 16k + (c ^ (k & 15)).  A
// transposing byte read runs as two 32-lane passes, each over 16 consecutive rows of one
// chunk, which this swizzle puts on 16 distinct 16-byte bank groups.
__device__ __forceinline__ int w8_swz(int k) { return k & 15; }

struct W8CopyPlan {
  uint32_t off[3];
};

__device__ __forceinline__ W8CopyPlan w8_offsets(const BigArgs& G, const WeightView& W, int m0, int wn0, int wn_end,
                                                 int w, int lane) {
  W8CopyPlan cp;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int e = 64 * (2 * w + i) + lane, r = e >> 2, c = (e & 3) ^ a4_swz(r);
    const int m = min(m0 + r, G.M - 1);
    cp.off[i] = (uint32_t)((m * G.lda + 8 * c) * 2);
  }
  const int e = 64 * w + lane, k = e >> 4, c = (e & 15) ^ w8_swz(k);
  const int n = min(wn0 + 16 * c, wn_end - 16);
  cp.off[2] = (uint32_t)(k * W.ld + n);
  return cp;
}

__device__ __forceinline__ void w8_issue(const BigArgs& G, const WeightView& W, const W8CopyPlan& cp, int k0,
                                         uint4* __restrict__ as, uint4* __restrict__ ws, int w) {
#pragma unroll
  for (int i = 0; i < 2; ++i) dma16_buf(G.A + k0, 0x7FFFFFF0u, cp.off[i], as + 64 * (2 * w + i));
  dma16_buf((const uint8_t*)W.w + (int64_t)k0 * W.ld, 0x7FFFFFF0u, cp.off[2], ws + 64 * w);
}

// B operand of 16-column tile nt of the wave, as one transposing byte read (w8_raw: lane (g, j)
// gets k = 8g .. 8g+7 of column 64*(w & 3) + 16*nt + j, byte b = row 8g + b) decoded with block
// scale s (w8_dec).
__device__ __forceinline__ i32x2w w8_raw(const uint4* __restrict__ ws, int nt, int w, int lane) {
  const int g = lane >> 4, j = lane & 15;
  const int k = 8 * g + (j >> 1);
  const int c = (4 * (w & 3) + nt) ^ w8_swz(k);
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2w*)((const char*)ws + (16 * k + c) * 16 + 8 * (j & 1)));
}

__device__ __forceinline__ bf16x8 w8_dec(i32x2w p, float s) {
  uint32_t o[4];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(p[q], false);
    const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(p[q], true);
    o[2 * q] = pack_bf16x2(lo[0] * s, lo[1] * s);
    o[2 * q + 1] = pack_bf16x2(hi[0] * s, hi[1] * s);
  }
  return as_bf16x8(make_uint4(o[0], o[1], o[2], o[3]));
}

// One K step, as big_step: this step's copies, then the matrix ops of the current stage column
// block by column block, each operand register refilled from the next stage `as1/ws1` right
// after its last op.  A B operand's byte read is issued one block before the block that last
// uses the register, and decoded (with the next step's block scale, from the scale table sc)
// right after that block, so no decode waits for a fresh read.  `pre` alone (no compute) reads
// and decodes all operands of the next stage: the first step's.  Every LDS access goes through
// restrict pointers.
__device__ __forceinline__ void w8_step(const BigArgs& G, const WeightView& W, const W8CopyPlan& cp, bool copy,
                                        int k_pf, bool compute, bool pre, int sc_idx, const float* __restrict__ sc,
                                        const uint4* __restrict__ as1, const uint4* __restrict__ ws1,
                                        uint4* __restrict__ as_nx, uint4* __restrict__ ws_nx, f32x4 (&acc)[8][4],
                                        bf16x8 (&af)[8], bf16x8 (&bf)[4], int w, int lane) {
  if (copy) w8_issue(G, W, cp, k_pf, as_nx, ws_nx, w);
  const float s1 = sc[sc_idx];
  if (compute) {
    i32x2w raw = w8_raw(ws1, 0, w, lane);
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      if (nt == 3) __builtin_amdgcn_s_waitcnt(0xC17F);  // lgkmcnt(1): all but the last B read
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) {
        acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[mt], bf[nt], acc[mt][nt], 0, 0, 0);
        if (nt == 3) {
          af[mt] = big_a(as1, mt, w, lane);
          __builtin_amdgcn_sched_barrier(0);  // each refill after its op: old and new never both live
        }
      }
      const i32x2w nxt = nt < 3 ? w8_raw(ws1, nt + 1, w, lane) : raw;
      bf[nt] = w8_dec(raw, s1);
      raw = nxt;
      __builtin_amdgcn_sched_barrier(0);
    }
  } else if (pre) {
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) af[mt] = big_a(as1, mt, w, lane);
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) bf[nt] = w8_dec(w8_raw(ws1, nt, w, lane), s1);
    __builtin_amdgcn_s_waitcnt(0xC07F);
  }
}

__global__ __launch_bounds__(512, 1) void gemm_w8_kernel(BigArgs G, EpiArgs E) {
  // kW8Stages stages of A (16 KB) and W (8 KB), also the epilogue's 128 KB bf16 tile
  __shared__ __attribute__((aligned(16))) uint4 smem[kW8Smem];
  __shared__ float scl[2][kW8MaxKBlocks];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n0 = blockIdx.x * kBigN, m0 = blockIdx.y * kBigM;
  const bool seg1 = n0 >= G.n_split;
  const WeightView W = seg1 ? G.W1 : G.W0;
  const int wn0 = seg1 ? n0 - G.n_split : n0, wn_end = seg1 ? G.N - G.n_split : G.n_split;
  const int kbeg = blockIdx.z * G.k_split, kend = min(G.K, kbeg + G.k_split);
  const int nsteps = (kend - kbeg) / kBigK;
  // block scales of the tile's two 128-column blocks over the K range (columns past the
  // segment, which are not stored, read the last block's scale)
  const int kg0 = kbeg / 128, nkb = (kend + 127) / 128 - kg0;
  for (int t = tid; t < 2 * nkb; t += 512) {
    const int lb = t / nkb, i = t - lb * nkb;
    const int nb = min(wn0 / 128 + lb, W.scale_ld - 1);
    scl[lb][i] = W.scale[(int64_t)(kg0 + i) * W.scale_ld + nb];
  }
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  lds_barrier();
  const W8CopyPlan cp = w8_offsets(G, W, m0, wn0, wn_end, w, lane);
  f32x4 acc[8][4];
#pragma unroll
  for (int mt = 0; mt < 8; ++mt)
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) acc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  bf16x8 af[8], bf[4];
#pragma unroll
  for (int i = 0; i < 8; ++i) af[i] = as_bf16x8(make_uint4(0u, 0u, 0u, 0u));
#pragma unroll
  for (int i = 0; i < 4; ++i) bf[i] = as_bf16x8(make_uint4(0u, 0u, 0u, 0u));
  // the wave's 64 columns lie in one 128-column block: row (w & 3) >> 1 of the scale table
  const int sc_row = ((w & 3) >> 1) * kW8MaxKBlocks - kg0;
  // iteration s: copies of step s + kW8Stages - 1, matrix ops of step s (s >= 0), operands of
  // step s + 1.  The first kW8Stages - 2 iterations (copies only) run before the loop, so that
  // the loop's liveness is that of the matrix steps alone.
  typedef __attribute__((address_space(3))) uint4 lds_uint4;
  for (int s = -(kW8Stages - 1); s < -1; ++s) {
    const int s_pf = s + kW8Stages - 1;
    if (s_pf < nsteps) {
      lds_uint4* base = (lds_uint4*)smem;
      w8_issue(G, W, cp, kbeg + s_pf * kBigK, (uint4*)(base + kW8StageA * s_pf),
               (uint4*)(base + kW8StageA * kW8Stages + kW8StageW * s_pf), w);
    }
  }
  for (int s = -1; s < nsteps; ++s) {
    {
      // steps s and s+1 in LDS: in the steady state the copies of the kW8Stages - 3 steps after
      // them stay in flight; near the end every copy is waited for
      constexpr int kAhead = kW8Copies * (kW8Stages - 3);
      if (s + kW8Stages - 2 < nsteps) __builtin_amdgcn_s_waitcnt(0x0F70 | (kAhead & 15) | ((kAhead >> 4) << 14));
      else __builtin_amdgcn_s_waitcnt(0x0F70);
      lds_barrier();
    }
    const int s_pf = s + kW8Stages - 1;
    const int b_pf = (s_pf + kW8Stages) % kW8Stages;
    const int b_1 = (s + 1 + kW8Stages) % kW8Stages;
    typedef __attribute__((address_space(3))) float lds_float;
    lds_uint4* base = (lds_uint4*)smem;
    lds_uint4 *a_1 = base + kW8StageA * b_1;
    lds_uint4 *w_1 = base + kW8StageA * kW8Stages + kW8StageW * b_1;
    lds_uint4 *a_nx = base + kW8StageA * b_pf, *w_nx = base + kW8StageA * kW8Stages + kW8StageW * b_pf;
    lds_float* sc = (lds_float*)&scl[0][0];
    asm volatile("" : "+s"(a_1), "+s"(w_1), "+s"(a_nx), "+s"(w_nx), "+s"(sc));
    // the next step's block scale (in the last step, a valid entry whose value is unused)
    const int sc_idx = sc_row + (kbeg + min(s + 1, nsteps - 1) * kBigK) / 128;
    w8_step(G, W, cp, s_pf < nsteps, kbeg + s_pf * kBigK, s >= 0, s == -1, sc_idx, (const float*)sc,
            (const uint4*)a_1, (const uint4*)w_1, (uint4*)a_nx, (uint4*)w_nx, acc, af, bf, w, lane);
  }
  big_epilogue<256, 256>(E, seg1 ? E.kind1 : E.kind, acc, (bf16_t*)&smem[0], G.M, G.N, G.C, G.ldc,
               (int64_t)blockIdx.z * G.split_stride, m0, n0, w, lane);
}

// ---------------------------------------------------------------------------------------------
// The same fp8-weight kernel with 128 x 128 tiles (4 waves of 64 x 64) for 64 < M <= 256: at
// M = 256 the 256 x 256 tile leaves too few workgroups (the v3 stage-1 projection 126, wq_b 96
// without a K split).  The W stage is [32 k][8 chunks of 16 columns], chunk c of row k at slot
// 8k + (c ^ ((k >> 1) & 7)): a 32-lane pass of the transposing byte read covers rows k0..k0+15
// of one chunk, the even rows in one 128-byte half of the 64 banks and the odd rows in the
// other, each half on 8 distinct 16-byte groups.
constexpr int kW8sStageA = 128 * 4, kW8sStageW = kBigK * 8;  // 16-byte chunks per stage
constexpr int kW8sSmem = kW8Stages * (kW8sStageA + kW8sStageW) > 2048 ? kW8Stages * (kW8sStageA + kW8sStageW) : 2048;

__device__ __forceinline__ int w8s_swz(int k) { return (k >> 1) & 7; }

__device__ __forceinline__ W8CopyPlan w8s_offsets(const BigArgs& G, const WeightView& W, int m0, int wn0, int wn_end,
                                                  int w, int lane) {
  W8CopyPlan cp;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int e = 64 * (2 * w + i) + lane, r = e >> 2, c = (e & 3) ^ a4_swz(r);
    const int m = min(m0 + r, G.M - 1);
    cp.off[i] = (uint32_t)((m * G.lda + 8 * c) * 2);
  }
  const int e = 64 * w + lane, k = e >> 3, c = (e & 7) ^ w8s_swz(k);
  const int n = min(wn0 + 16 * c, wn_end - 16);
  cp.off[2] = (uint32_t)(k * W.ld + n);
  return cp;
}

// A rows 64*(w >> 1) + 16*mt + j; B columns 64*(w & 1) + 16*nt + j (k = 8g .. 8g+7).
__device__ __forceinline__ bf16x8 w8s_a(const uint4* __restrict__ as, int mt, int w, int lane) {
  const int r = 64 * (w >> 1) + 16 * mt + (lane & 15);
  return as_bf16x8(as[4 * r + ((lane >> 4) ^ a4_swz(r))]);
}

__device__ __forceinline__ i32x2w w8s_raw(const uint4* __restrict__ ws, int nt, int w, int lane) {
  const int g = lane >> 4, j = lane & 15;
  const int k = 8 * g + (j >> 1);
  const int c = (4 * (w & 1) + nt) ^ w8s_swz(k);
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2w*)((const char*)ws + (8 * k + c) * 16 + 8 * (j & 1)));
}

// One K step, as w8_step (16 matrix ops per wave, column block by column block, operands
// refilled from the next stage right after their last use).
__device__ __forceinline__ void w8s_step(const BigArgs& G, const WeightView& W, const W8CopyPlan& cp, bool copy,
                                         int k_pf, bool compute, bool pre, int sc_idx, const float* __restrict__ sc,
                                         const uint4* __restrict__ as1, const uint4* __restrict__ ws1,
                                         uint4* __restrict__ as_nx, uint4* __restrict__ ws_nx, f32x4 (&acc)[4][4],
                                         bf16x8 (&af)[4], bf16x8 (&bf)[4], int w, int lane) {
  if (copy) {
#pragma unroll
    for (int i = 0; i < 2; ++i) dma16_buf(G.A + k_pf, 0x7FFFFFF0u, cp.off[i], as_nx + 64 * (2 * w + i));
    dma16_buf((const uint8_t*)W.w + (int64_t)k_pf * W.ld, 0x7FFFFFF0u, cp.off[2], ws_nx + 64 * w);
  }
  const float s1 = sc[sc_idx];
  if (compute) {
    i32x2w raw = w8s_raw(ws1, 0, w, lane);
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      if (nt == 3) __builtin_amdgcn_s_waitcnt(0xC17F);  // lgkmcnt(1): all but the last B read
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[mt], bf[nt], acc[mt][nt], 0, 0, 0);
        if (nt == 3) {
          af[mt] = w8s_a(as1, mt, w, lane);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      const i32x2w nxt = nt < 3 ? w8s_raw(ws1, nt + 1, w, lane) : raw;
      bf[nt] = w8_dec(raw, s1);
      raw = nxt;
      __builtin_amdgcn_sched_barrier(0);
    }
  } else if (pre) {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) af[mt] = w8s_a(as1, mt, w, lane);
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) bf[nt] = w8_dec(w8s_raw(ws1, nt, w, lane), s1);
    __builtin_amdgcn_s_waitcnt(0xC07F);
  }
}

__global__ __launch_bounds__(256) void gemm_w8s_kernel(BigArgs G, EpiArgs E) {
  __shared__ __attribute__((aligned(16))) uint4 smem[kW8sSmem];
  __shared__ float scl[kW8MaxKBlocks];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n0 = blockIdx.x * 128, m0 = blockIdx.y * 128;
  const bool seg1 = n0 >= G.n_split;
  const WeightView W = seg1 ? G.W1 : G.W0;
  const int wn0 = seg1 ? n0 - G.n_split : n0, wn_end = seg1 ? G.N - G.n_split : G.n_split;
  const int kbeg = blockIdx.z * G.k_split, kend = min(G.K, kbeg + G.k_split);
  const int nsteps = (kend - kbeg) / kBigK;
  // the tile's block scales over the K range (one 128-column block)
  const int kg0 = kbeg / 128, nkb = (kend + 127) / 128 - kg0;
  const int nb = min(wn0 / 128, W.scale_ld - 1);
  for (int t = tid; t < nkb; t += 256) scl[t] = W.scale[(int64_t)(kg0 + t) * W.scale_ld + nb];
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  lds_barrier();
  const W8CopyPlan cp = w8s_offsets(G, W, m0, wn0, wn_end, w, lane);
  f32x4 acc[4][4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) acc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  bf16x8 af[4], bf[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) af[i] = bf[i] = as_bf16x8(make_uint4(0u, 0u, 0u, 0u));
  typedef __attribute__((address_space(3))) uint4 lds_uint4;
  typedef __attribute__((address_space(3))) float lds_float;
  // copy-only iterations first (as in gemm_w8_kernel), then step -1 (operands of step 0) and
  // the matrix steps
  for (int s = -(kW8Stages - 1); s < -1; ++s) {
    const int s_pf = s + kW8Stages - 1;
    if (s_pf < nsteps) {
      lds_uint4* base = (lds_uint4*)smem;
      uint4* an = (uint4*)(base + kW8sStageA * s_pf);
      uint4* wn = (uint4*)(base + kW8sStageA * kW8Stages + kW8sStageW * s_pf);
#pragma unroll
      for (int i = 0; i < 2; ++i) dma16_buf(G.A + kbeg + s_pf * kBigK, 0x7FFFFFF0u, cp.off[i], an + 64 * (2 * w + i));
      dma16_buf((const uint8_t*)W.w + (int64_t)(kbeg + s_pf * kBigK) * W.ld, 0x7FFFFFF0u, cp.off[2], wn + 64 * w);
    }
  }
  for (int s = -1; s < nsteps; ++s) {
    {
      constexpr int kAhead = kW8Copies * (kW8Stages - 3);
      if (s + kW8Stages - 2 < nsteps) __builtin_amdgcn_s_waitcnt(0x0F70 | (kAhead & 15) | ((kAhead >> 4) << 14));
      else __builtin_amdgcn_s_waitcnt(0x0F70);
      lds_barrier();
    }
    const int s_pf = s + kW8Stages - 1;
    const int b_pf = (s_pf + kW8Stages) % kW8Stages;
    const int b_1 = (s + 1 + kW8Stages) % kW8Stages;
    lds_uint4* base = (lds_uint4*)smem;
    lds_uint4 *a_1 = base + kW8sStageA * b_1;
    lds_uint4 *w_1 = base + kW8sStageA * kW8Stages + kW8sStageW * b_1;
    lds_uint4 *a_nx = base + kW8sStageA * b_pf, *w_nx = base + kW8sStageA * kW8Stages + kW8sStageW * b_pf;
    lds_float* sc = (lds_float*)&scl[0];
    asm volatile("" : "+s"(a_1), "+s"(w_1), "+s"(a_nx), "+s"(w_nx), "+s"(sc));
    const int sc_idx = (kbeg + min(s + 1, nsteps - 1) * kBigK) / 128 - kg0;
    w8s_step(G, W, cp, s_pf < nsteps, kbeg + s_pf * kBigK, s >= 0, s == -1, sc_idx, (const float*)sc,
             (const uint4*)a_1, (const uint4*)w_1, (uint4*)a_nx, (uint4*)w_nx, acc, af, bf, w, lane);
  }
  big_epilogue<128, 128>(E, seg1 ? E.kind1 : E.kind, acc, (bf16_t*)&smem[0], G.M, G.N, G.C, G.ldc,
                         (int64_t)blockIdx.z * G.split_stride, m0, n0, w, lane);
}

bool w8s_ok(const Dims& d, int M, int N, int K, int n_split, int64_t lda, int k_split) {
  return d.wk == W_FP8 && M > 64 && M <= 256 && K % kBigK == 0 && k_split % 128 == 0 &&
         (k_split + 127) / 128 + 1 <= kW8MaxKBlocks && (n_split >= N || n_split % 128 == 0) && N % 16 == 0 &&
         (n_split >= N || (N - n_split) % 16 == 0) && ((int64_t)M * lda + K) * 2 < 0x7FFFFFF0LL;
}

bool w8_ok(const Dims& d, int M, int N, int K, int n_split, int64_t lda, int k_split) {
  return d.wk == W_FP8 && M > 64 && M <= 1024 && K % kBigK == 0 && k_split % kBigK == 0 &&
         (k_split + 127) / 128 + 1 <= kW8MaxKBlocks && (n_split >= N || n_split % kBigN == 0) && N % 16 == 0 &&
         (n_split >= N || (N - n_split) % 16 == 0) && ((int64_t)M * lda + K) * 2 < 0x7FFFFFF0LL;
}

bool big_ok(const Dims& d, int M, int N, int K, int n_split, int64_t lda) {
  // activation offsets are 32-bit byte offsets from the K step's column
  return d.wk == W_BF16 && M > 512 && K % kBigK == 0 && (n_split >= N || n_split % kBigN == 0) && N % 8 == 0 &&
         (n_split >= N || (N - n_split) % 8 == 0) && ((int64_t)M * lda + K) * 2 < 0x7FFFFFF0LL;
}

struct Plan {
  int bm, splits, k_split;
  bool w8s = false;  // fp8 weights, 64 < M <= 256: gemm_w8s_kernel's 128 x 128 tiles
};

Plan plan(int M, int N, int K, int wk) {
  Plan p;
  if (M > 512 && M <= 1024 && wk == W_BF16) {  // 256 x 256 tiles, few of them: K split in 1, 2 or 4
    // ranges (>= 1024 k each), whichever gives the fewest rounds of 256 workgroups per unit of
    // work (the partial sums of M <= 1024 rows are small)
    p.bm = 128;
    const int64_t tiles = (int64_t)((N + 255) / 256) * ((M + 255) / 256);
    int best = 1;
    double best_t = (double)((tiles + 255) / 256);
    for (int sp = 2; sp <= 4; sp *= 2) {
      if (K % (64 * sp) != 0 || K / sp < 1024) break;
      const double t = (double)((tiles * sp + 255) / 256) / sp;
      if (t < best_t) {
        best = sp;
        best_t = t;
      }
    }
    p.splits = best;
    p.k_split = K / best;
    return p;
  }
  if (M > 1024) {  // prefill shapes (256 x 256 tiles): whole K per workgroup, unless the
    // tile count leaves most of a last round of one workgroup per CU idle and K is long:
    // then two K ranges (partial sums) halve the rounds' length
    p.bm = 128;
    p.splits = 1;
    p.k_split = K;
    const int64_t tiles = (int64_t)((N + 255) / 256) * ((M + 255) / 256);
    const double r1 = (double)((tiles + 255) / 256), r2 = (double)((2 * tiles + 255) / 256) / 2.0;
    if (K >= 2048 && K % 64 == 0 && r2 <= 0.75 * r1) {
      p.splits = 2;
      p.k_split = K / 2;
    }
    return p;
  }
  if (wk == W_FP8 && M > 64) {  // gemm_w8_kernel (256 x 256 tiles): K spread over the CUs, but
    // >= kW8MinKSplit k per split, so that the fp32 partial sums stay a fraction of the weights
    auto split_k = [&](int tiles) {
      int splits = max(1, 256 / tiles);
      while (splits > 1 && K / splits < kW8MinKSplit) --splits;
      p.k_split = ((K + splits - 1) / splits + 127) / 128 * 128;
      p.splits = (K + p.k_split - 1) / p.k_split;
    };
    p.bm = 256;
    split_k(((N + kBigN - 1) / kBigN) * ((M + kBigM - 1) / kBigM));
    // up to 256 rows, when those tiles leave the CUs short of work (fewer than 224 workgroups),
    // gemm_w8s_kernel's 128 x 128 tiles instead (v3 at B = 256: stage-1 126 -> 238 workgroups,
    // wq_b 192 -> 384 without a K split, so its RoPE runs in the epilogue; wo stays at 252)
    if (M <= 256 && (int64_t)((N + kBigN - 1) / kBigN) * ((M + kBigM - 1) / kBigM) * p.splits < 224) {
      p.w8s = true;
      split_k(((N + 127) / 128) * ((M + 127) / 128));
    }
    return p;
  }
  p.bm = M <= 64 ? 64 : 128;
  const int tiles = ((N + BN - 1) / BN) * ((M + p.bm - 1) / p.bm);
  // skinny shapes: spread K over as many workgroups as there are CUs, one each (a workgroup that
  // streams a longer K range beats two sharing a CU, and fewer splits mean fewer partial sums),
  // keeping >= 128 k per split; with one split the consumer's epilogue runs in the GEMM itself
  int splits = max(1, 256 / tiles);
  while (splits > 1 && K / splits < 128) --splits;
  p.k_split = ((K + splits - 1) / splits + BK - 1) / BK * BK;
  p.splits = (K + p.k_split - 1) / p.k_split;
  return p;
}

template <int BM, int WM, int WN>
hipError_t launch(const Dims& d, const void* A, int64_t lda, const WeightView& W0, const WeightView& W1, int n_split,
                  float* C, int64_t ldc, int M, int N, int K, int k_split, int splits, int64_t split_stride,
                  const EpiArgs& E, hipStream_t s) {
  dim3 grid((N + BN - 1) / BN, (M + BM - 1) / BM, splits);
  if (BM == 64 && dec_ok(d, M, N, K, k_split, n_split, lda, C, ldc, split_stride)) {
    DecArgs G{(const bf16_t*)A, lda, W0, W1, n_split, C, ldc, M, N, K, k_split, split_stride};
    gemm_dec_kernel<<<grid, 256, 0, s>>>(G, E);
    return hipGetLastError();
  }
  if (d.wk == W_FP8)
    gemm_kernel<BM, WM, WN, W_FP8><<<grid, 256, 0, s>>>((const bf16_t*)A, lda, W0, W1, n_split, C, ldc, M, N, K,
                                                        k_split, split_stride, E);
  else
    gemm_kernel<BM, WM, WN, W_BF16><<<grid, 256, 0, s>>>((const bf16_t*)A, lda, W0, W1, n_split, C, ldc, M, N, K,
                                                         k_split, split_stride, E);
  return hipGetLastError();
}

hipError_t launch_plan(const Plan& p, const Dims& d, const void* A, int64_t lda, const WeightView& W0,
                       const WeightView& W1, int n_split, float* C, int64_t ldc, int M, int N, int K, int64_t stride,
                       const EpiArgs& E, hipStream_t s) {
  return p.bm == 64 ? launch<64, 1, 4>(d, A, lda, W0, W1, n_split, C, ldc, M, N, K, p.k_split, p.splits, stride, E, s)
                    : launch<128, 2, 2>(d, A, lda, W0, W1, n_split, C, ldc, M, N, K, p.k_split, p.splits, stride, E, s);
}

// ---------------------------------------------------------------------------------------------
// fp8 variant of the large-M kernel: A holds E4M3FN codes with one power-of-two (E8M0) scale
// per row and 128 columns, W E4M3FN codes with fp32 128 x 128 block scales that must be powers
// of two (the compact 8-bit exponent scales of the NKI context-encoding kernel's MX fp8
// weights).  Each K step of 128 is one 16x16x128 fp8 matrix op per output block, which applies
// both scales itself (a per-lane E8M0 operand: the row's activation exponent, the block's
// weight exponent).  Same 256 x 256 tile and 8-wave layout as gemm_big_kernel, hence the
// same epilogue; two 64 KB stages.
//   Operand layout (probed on gfx950): the op sums A[r][kappa(g, t)] * B[kappa(g, t)][c] over
//   the 32 bytes t of lane group g = lane / 16 with one bijection kappa for both operands, so
//   any k order works as long as A and B use the same one: here k = 32 g + t.  A lane (row
//   lane % 16) reads its 32 bytes as two 16-byte chunks; a B lane (column lane % 16) gets
//   k = 32 g + 8 q + b from four ds_read_b64_tr_b8 (lanes 2b, 2b + 1 of a group address row b
//   of an 8 x 16-byte tile, lane i receives its column i).  The scale of row r for the
//   op's k block b comes from lane 16 b + r, so every lane passes its own row's exponent.
constexpr int kF8K = 128;
constexpr int kF8Copies = 8;  // per wave per stage: 4 activation + 4 weight copies of 1 KB

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;

// A stage [256 rows][8 chunks of 16 B]: chunk c of row r at slot 8r + (c ^ ((r >> 1) & 5));
// W stage [128 k][16 chunks]: chunk c of row k at slot 16k + (c ^ f8w_swz(k)).  Both keep the
// operand reads' lane passes on distinct banks.
__device__ __forceinline__ int f8a_swz(int r) { return (r >> 1) & 5; }
__device__ __forceinline__ int f8w_swz(int k) { return (k & 7) | (((k >> 5) & 1) << 3); }

// Activation exponents (f8_exp_order) are grouped so that the 8 rows a lane needs, 16 mt + j
// for mt = 0..7 of one 128-row half of the tile, are one 8-byte load.
struct F8Args {
  const uint8_t* A;  // E4M3FN codes [M, K] (row stride lda bytes)
  int64_t lda;
  const uint8_t* Ae;  // E8M0 exponents [K / 128][f8_rows_pad(M)], f8_exp_order
  WeightView W0, W1;
  int n_split;
  float* C;
  int64_t ldc;
  int M, N, K;
  int k_split;
  int64_t split_stride;
};

// acc += (A * 2^(byte SEL of sa - 127)) (B * 2^(sb - 127)) for one 16x16x128 E4M3 block
template <int SEL>
__device__ __forceinline__ f32x4 f8_mma(const i32x8& a, const i32x8& b, const f32x4& c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, SEL, sa, 0, sb);
}

// A lane's byte offsets of its copies within a K step (four activation, four weight), from
// the step's first column of A and first row of W: the same for every step of a tile.
struct F8CopyPlan {
  uint32_t off[8];
};

__device__ __forceinline__ F8CopyPlan f8_offsets(const F8Args& G, const WeightView& W, int m0, int wn0, int wn_end,
                                                 int w, int lane) {
  F8CopyPlan cp;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = 64 * (4 * w + i) + lane, r = e >> 3, c = (e & 7) ^ f8a_swz(r);
    const int m = min(m0 + r, G.M - 1);
    cp.off[i] = (uint32_t)(m * G.lda + 16 * c);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = 64 * (4 * w + i) + lane, k = e >> 4, c = (e & 15) ^ f8w_swz(k);
    const int n = min(wn0 + 16 * c, wn_end - 16);
    cp.off[4 + i] = (uint32_t)(k * W.ld + n);
  }
  return cp;
}

__device__ __forceinline__ void f8_issue(const F8Args& G, const WeightView& W, const F8CopyPlan& cp, int k0,
                                         uint4* __restrict__ as, uint4* __restrict__ ws, int w) {
  const uint8_t* ab = (const uint8_t*)G.A + k0;
#pragma unroll
  for (int i = 0; i < 4; ++i) dma16_buf(ab, 0x7FFFFFF0u, cp.off[i], as + 64 * (4 * w + i));
  const uint8_t* wb = (const uint8_t*)W.w + (int64_t)k0 * W.ld;
#pragma unroll
  for (int i = 0; i < 4; ++i) dma16_buf(wb, 0x7FFFFFF0u, cp.off[4 + i], ws + 64 * (4 * w + i));
}

__device__ __forceinline__ void f8_step(const F8Args& G, const WeightView& W, const F8CopyPlan& cp, int m0, bool copy,
                                        int k_pf, const uint4* __restrict__ as, const uint4* __restrict__ ws,
                                        uint4* __restrict__ as_nx, uint4* __restrict__ ws_nx, f32x4 (&acc)[8][4],
                                        uint2 sa, int sb, uint2& sa_nx, uint32_t& sw_nx, int nb, int w, int lane) {
  const int g = lane >> 4, j = lane & 15, wm = w >> 2, wn = w & 3;
  if (copy) {
    // exponents of the next step, a step ahead of their use: 8 activation rows of the lane
    // (4 per register) and the weight block scale of the wave
    const int kg = k_pf / kF8K;
    const int64_t m_pad = f8_rows_pad(G.M);
    sa_nx = *(const uint2*)(G.Ae + f8_exp_order(kg, m0 + 128 * wm + j, m_pad));
    sw_nx = __float_as_uint(W.scale[(int64_t)kg * W.scale_ld + nb]);
    f8_issue(G, W, cp, k_pf, as_nx, ws_nx, w);
  }
  i32x8 bfr[4];
  const char* wsb = (const char*)ws;
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    const int c = 4 * wn + nt;
    i32x2 p[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int k = 32 * g + 8 * q + (j >> 1);
      p[q] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(wsb + (16 * k + (c ^ f8w_swz(k))) * 16 + 8 * (j & 1)));
    }
    bfr[nt] = i32x8{p[0][0], p[0][1], p[1][0], p[1][1], p[2][0], p[2][1], p[3][0], p[3][1]};
  }
#pragma unroll
  for (int mt = 0; mt < 8; ++mt) {
    const int r = 128 * wm + 16 * mt + j;
    const uint4 lo = as[8 * r + ((2 * g) ^ f8a_swz(r))], hi = as[8 * r + ((2 * g + 1) ^ f8a_swz(r))];
    const i32x8 af = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    const int sreg = mt < 4 ? (int)sa.x : (int)sa.y;
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      switch (mt & 3) {  // byte of the exponent register: an immediate of the instruction
        case 0: acc[mt][nt] = f8_mma<0>(af, bfr[nt], acc[mt][nt], sreg, sb); break;
        case 1: acc[mt][nt] = f8_mma<1>(af, bfr[nt], acc[mt][nt], sreg, sb); break;
        case 2: acc[mt][nt] = f8_mma<2>(af, bfr[nt], acc[mt][nt], sreg, sb); break;
        default: acc[mt][nt] = f8_mma<3>(af, bfr[nt], acc[mt][nt], sreg, sb); break;
      }
    }
  }
}

__global__ __launch_bounds__(512, 1) void gemm_f8_kernel(F8Args G, EpiArgs E) {
  __shared__ __attribute__((aligned(16))) uint4 smem[2][4096];  // per stage: A 2048 + W 2048 chunks
  const int tid = threadIdx.x, lane = tid & 63, j = lane & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = w >> 2, wn = w & 3;
  const int n0 = blockIdx.x * kBigN, m0 = blockIdx.y * kBigM;
  const bool seg1 = n0 >= G.n_split;
  const WeightView W = seg1 ? G.W1 : G.W0;
  const int wn0 = seg1 ? n0 - G.n_split : n0, wn_end = seg1 ? G.N - G.n_split : G.n_split;
  const int kbeg = blockIdx.z * G.k_split;
  const int nsteps = (min(G.K, kbeg + G.k_split) - kbeg) / kF8K;
  // the wave's 64 columns lie in one 128-column scale block (waves past the segment's end,
  // whose columns are not stored, read the last block's scale)
  const int nb = min((wn0 + 64 * wn) / 128, W.scale_ld - 1);
  const F8CopyPlan cp = f8_offsets(G, W, m0, wn0, wn_end, w, lane);
  f32x4 acc[8][4];
#pragma unroll
  for (int mt = 0; mt < 8; ++mt)
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) acc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  unsigned bad = 0;  // a weight scale that is not a positive power of two
  uint2 sa = make_uint2(0, 0), sa_nx = make_uint2(0, 0);
  uint32_t sw = 0, sw_nx = 0;
  if (nsteps > 0) {
    typedef __attribute__((address_space(3))) uint4 lds_uint4;
    lds_uint4 *a0 = (lds_uint4*)&smem[0][0], *w0 = (lds_uint4*)&smem[0][2048];
    asm volatile("" : "+s"(a0), "+s"(w0));
    const int kg = kbeg / kF8K;
    const int64_t m_pad = f8_rows_pad(G.M);
    sa = *(const uint2*)(G.Ae + f8_exp_order(kg, m0 + 128 * wm + j, m_pad));
    sw = __float_as_uint(W.scale[(int64_t)kg * W.scale_ld + nb]);
    f8_issue(G, W, cp, kbeg, (uint4*)a0, (uint4*)w0, w);
  }
  for (int s = 0; s < nsteps; ++s) {
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's copies of step s
    lds_barrier();                       // every wave's copies landed; stage (s + 1) % 2 is free
    const bool more = s + 1 < nsteps;
    typedef __attribute__((address_space(3))) uint4 lds_uint4;
    lds_uint4 *a_cur = (lds_uint4*)&smem[s & 1][0], *w_cur = (lds_uint4*)&smem[s & 1][2048];
    lds_uint4 *a_nx = (lds_uint4*)&smem[(s + 1) & 1][0], *w_nx = (lds_uint4*)&smem[(s + 1) & 1][2048];
    asm volatile("" : "+s"(a_cur), "+s"(w_cur), "+s"(a_nx), "+s"(w_nx));
    const int sb = (int)((sw >> 23) & 0xFF);
    bad |= (sw & 0x807FFFFFu) | (sb == 0 || sb == 0xFF);
    f8_step(G, W, cp, m0, more, kbeg + (s + 1) * kF8K, (const uint4*)a_cur, (const uint4*)w_cur,
            (uint4*)a_nx, (uint4*)w_nx, acc, sa, sb, sa_nx, sw_nx, nb, w, lane);
    sa = sa_nx;
    sw = sw_nx;
  }
  if (bad) {  // weight scales outside the supported form poison the tile instead of giving wrong numbers
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) acc[mt][nt] = f32x4{NAN, NAN, NAN, NAN};
  }
  big_epilogue<256, 256>(E, seg1 ? E.kind1 : E.kind, acc, (bf16_t*)&smem[0][0], G.M, G.N, G.C, G.ldc,
               (int64_t)blockIdx.z * G.split_stride, m0, n0, w, lane);
}

bool f8_ok(const Dims& d, int M, int N, int K, int n_split, int k_split) {
  return d.wk == W_FP8 && M > 1024 && K % kF8K == 0 && k_split % kF8K == 0 &&
         (n_split >= N || n_split % kBigN == 0) && N % 16 == 0 && (n_split >= N || (N - n_split) % 16 == 0) &&
         (int64_t)M * K + K < 0x7FFFFFF0LL;
}

}  // namespace

bool fast_proj_supported(const Dims& d) {
  // every K and N is a multiple of the 16-byte load width (16 columns for fp8 bytes)
  const int q = d.wk == W_FP8 ? 16 : 8;
  return d.act == 1 && (d.wk == W_BF16 || d.wk == W_FP8) && d.D % q == 0 && d.Lq % q == 0 && d.Lkv % 8 == 0 &&
         (d.Lkv + d.dr) % q == 0 && (d.H * (d.dn + d.dr)) % q == 0 && (d.H * (d.dn + d.dv)) % q == 0 &&
         (d.H * d.dv) % 8 == 0;
}

size_t fast_gemm_out_bytes(const Dims& d, int M, int N, int K) {
  if (M <= 0 || N <= 0 || K <= 0) return 0;
  return (size_t)plan(M, N, K, d.wk).splits * M * N * sizeof(float);
}

bool fast_gemm_fusable(const Dims& d, int M, int N, int K, int n_split, int kind) {
  if (!fast_proj_supported(d) || kind == GemmEpilogue::PARTIALS || M <= 0 || N <= 0 || K <= 0) return false;
  const bool aligned = n_split >= N || n_split % BN == 0;
  // the query consumer pairs columns 2i, 2i+1 of each head's rope part within a lane pair
  const bool pairs_ok = d.dn % 2 == 0 && (d.dn + d.dr) % 2 == 0;
  // the k/v consumer stores 16-byte chunks of 8 columns, which must stay inside one head part
  const bool kv_ok = d.dn % 8 == 0 && d.dv % 8 == 0 && (d.dn + d.dr) % 8 == 0;
  return plan(M, N, K, d.wk).splits == 1 && aligned && (kind != GemmEpilogue::QUERY || pairs_ok) &&
         (kind != GemmEpilogue::KV || kv_ok);
}

hipError_t fast_gemm(const Dims& d, const void* A, int64_t lda, const WeightView& W0, int n_split, const WeightView& W1,
                     int M, int N, int K, float* out, Partials* res, const GemmEpilogue* epi, bool* fused,
                     hipStream_t s) {
  const Plan p = plan(M, N, K, d.wk);
  const int64_t stride = (int64_t)M * N;
  *res = Partials{out, p.splits, stride, N};
  if (fused) *fused = false;
  if (M <= 0 || N <= 0 || K <= 0) return hipSuccess;
  EpiArgs E{GemmEpilogue::PARTIALS, nullptr, nullptr, nullptr, nullptr, d.H, d.dn, d.dr, d.dv};
  const bool aligned = n_split >= N || n_split % BN == 0;
  if (epi && epi->seg1_partials) {
    // W0's tiles to the query consumer, W1's as partial sums: the large-tile kernel, K unsplit
    const bool pairs_ok = d.dn % 2 == 0 && (d.dn + d.dr) % 2 == 0;
    if (epi->kind == GemmEpilogue::QUERY && pairs_ok && n_split < N && n_split % kBigN == 0 && n_split % 8 == 0 &&
        p.splits == 1 && big_ok(d, M, N, K, n_split, lda)) {
      E.kind = GemmEpilogue::QUERY;
      E.kind1 = GemmEpilogue::PARTIALS;
      E.y = (bf16_t*)epi->y;
      E.ldy = n_split;
      E.cosT = epi->cosT;
      E.sinT = epi->sinT;
      if (fused) *fused = true;
    }
  } else if (epi && fast_gemm_fusable(d, M, N, K, n_split, epi->kind)) {
    E.kind = E.kind1 = epi->kind;
    E.y = (bf16_t*)epi->y;
    E.y2 = (bf16_t*)epi->y2;
    E.cosT = epi->cosT;
    E.sinT = epi->sinT;
    if (fused) *fused = true;
  }
  if (p.w8s && w8s_ok(d, M, N, K, n_split, lda, p.k_split)) {
    BigArgs G{(const bf16_t*)A, lda, W0, W1, n_split < N ? n_split : N, out, N, M, N, K, p.k_split, stride};
    gemm_w8s_kernel<<<dim3((N + 127) / 128, (M + 127) / 128, p.splits), 256, 0, s>>>(G, E);
    return hipGetLastError();
  }
  if (p.bm == kBigM && !p.w8s && w8_ok(d, M, N, K, n_split, lda, p.k_split)) {
    BigArgs G{(const bf16_t*)A, lda, W0, W1, n_split < N ? n_split : N, out, N, M, N, K, p.k_split, stride};
    gemm_w8_kernel<<<dim3((N + kBigN - 1) / kBigN, (M + kBigM - 1) / kBigM, p.splits), 512, 0, s>>>(G, E);
    return hipGetLastError();
  }
  if (big_ok(d, M, N, K, n_split, lda)) {
    BigArgs G{(const bf16_t*)A, lda, W0, W1, n_split < N ? n_split : N, out, N, M, N, K, p.k_split, stride};
    gemm_big_kernel<<<dim3((N + kBigN - 1) / kBigN, (M + kBigM - 1) / kBigM, p.splits), 512, 0, s>>>(G, E);
    return hipGetLastError();
  }
  if (aligned) return launch_plan(p, d, A, lda, W0, W1, n_split < N ? n_split : N, out, N, M, N, K, stride, E, s);
  // segments not aligned to the column tile: one launch each, same split plan and partial layout
  hipError_t e = launch_plan(p, d, A, lda, W0, W0, n_split, out, N, M, n_split, K, stride, E, s);
  if (e != hipSuccess) return e;
  return launch_plan(p, d, A, lda, W1, W1, N - n_split, out + n_split, N, M, N - n_split, K, stride, E, s);
}

bool fast_gemm_f8_ok(const Dims& d, int M, int N, int K, int n_split) {
  if (!fast_proj_supported(d) || M <= 0 || N <= 0 || K <= 0) return false;
  return f8_ok(d, M, N, K, n_split, plan(M, N, K, d.wk).k_split);
}

hipError_t fast_gemm_f8(const Dims& d, const uint8_t* A8, const uint8_t* Ae, const WeightView& W0, int n_split,
                        const WeightView& W1, int M, int N, int K, float* out, Partials* res,
                        const GemmEpilogue* epi, bool* fused, hipStream_t s) {
  const Plan p = plan(M, N, K, d.wk);
  const int64_t stride = (int64_t)M * N;
  *res = Partials{out, p.splits, stride, N};
  if (fused) *fused = false;
  if (!fast_gemm_f8_ok(d, M, N, K, n_split)) return hipErrorInvalidValue;
  EpiArgs E{GemmEpilogue::PARTIALS, nullptr, nullptr, nullptr, nullptr, d.H, d.dn, d.dr, d.dv};
  if (epi && !epi->seg1_partials && fast_gemm_fusable(d, M, N, K, n_split, epi->kind)) {
    E.kind = E.kind1 = epi->kind;
    E.y = (bf16_t*)epi->y;
    E.y2 = (bf16_t*)epi->y2;
    E.cosT = epi->cosT;
    E.sinT = epi->sinT;
    if (fused) *fused = true;
  }
  F8Args G{A8, K, Ae, W0, W1, n_split < N ? n_split : N, out, N, M, N, K, p.k_split, stride};
  gemm_f8_kernel<<<dim3((N + kBigN - 1) / kBigN, (M + kBigM - 1) / kBigM, p.splits), 512, 0, s>>>(G, E);
  return hipGetLastError();
}

}  // namespace mla
