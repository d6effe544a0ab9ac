// The layer-step for batches of up to 64 tokens, as five launches.
//
// At tens of tokens an expert is shared by many tokens (the hot-expert case:
// 64 tokens over 32 experts, 16 tokens each), and a row-at-a-time GEMV that
// re-reads every token's activations for every 16 bytes of weights runs out
// of vector issue long before HBM runs out of bandwidth.  Every contraction
// whose weights are shared by 16 or more tokens therefore runs on the matrix
// cores (v_mfma_f32_16x16x32_bf16, fp32 accumulation); experts with fewer
// tokens keep the VALU GEMV.  The decode step is the same as in the
// single-launch kernel (wireai.ir "vLLM's speed jump on NVIDIA Blackwell
// servers; record 842 tokens/s for Kimi K3", section "Four key changes behind
// the jump", bullets 1-3: input projection, out-projection into the residual
// and norm, router before the shared and routed experts).
//
// Launches (all on the caller's stream; data passes through L2/HBM):
//  1 proj_b    64 rows of Wo per workgroup, K = Do split over the 4 waves:
//                r1 = r + attn Wo^T -> resid_out, hg = g r1, per-workgroup
//                sums of r1^2.
//              64 rows of Wqkv per workgroup, K = H split over 8 workgroups
//                (4 when H % 1024 != 0) x 4 waves: partial qkv sums.
//              Operands loaded as whole cache lines, relaid through LDS.
//  2 router_b  fp32 router dot products d[t, e] = hg[t] . Wr[e] on MFMA
//              (v_mfma_f32_16x16x4_f32), 48 experts x 256 K per workgroup,
//              tiles ordered so each XCD's workgroups share hg K chunks,
//              operands staged through LDS; also sums the qkv partials
//              (fixed order) -> qkv.
//  3 topk_b    one workgroup per token: 1/rms, h = hg / rms (fp32 and bf16
//              hi + lo planes), logits l = d / rms, top-k by repeated wave
//              arg-max (descending, ties to the lower expert id), weights
//              s / sum s with s = sigmoid(l).  The last workgroup to finish
//              builds the per-expert token lists (active experts ascending,
//              tokens ascending inside an expert) with wave prefix sums.
//  4 gateup_b  a[p, f] = silu(W1[e, f] . h[t_p]) * (W3[e, f] . h[t_p]):
//              matrix-core units (64 rows of W1 and W3 x a 16-token chunk
//              x a K chunk) cut into one contiguous run per workgroup, two
//              workgroups per CU, K chunks combined by the last to arrive;
//              then the VALU items of experts with fewer than 16 tokens.
//  5 down_b    y[t, i] = S2[i] . a_s[t] + sum_p w_p W2[e_p, i] . a[p]:
//              units (64 rows of y, one expert) cut into one contiguous run
//              per workgroup, each expert's activations staged once in LDS,
//              per-workgroup y tiles added in a fixed order by the last.
//
// MFMA operands.  x, attn and the weights are bf16 already.  h and the SwiGLU
// activations are fp32; each is split as x = hi + lo with hi = x truncated
// to bf16 (x - hi is exact) and lo = bf16(x - hi), and both halves are
// multiplied into the same accumulator, which keeps about 16 significant
// bits of x (relative error below 2^-16) against the weights' exact bf16.
//
// Weight loads.  A matrix-core operand fragment is 16 rows x 64 bytes per
// load instruction (the next 64 bytes of each row follow in the next K
// step), and these kernels read weights with ordinary cached loads: on this
// pattern they stream measurably faster than non-temporal loads.  That
// pattern touches 16 half-used cache lines per instruction, so the weights
// are loaded as whole lines instead (4 or 8 rows x 256 or 128 contiguous
// bytes per instruction) and moved into the fragment layout through LDS:
// by each wave through its own rows in the projections, gate/up and down,
// and by global-to-LDS loads in the router.
//
// Every output element is produced by one thread, in an order that depends
// only on the shapes, so results are bit-identical from run to run.
#include "common.h"
#include "kernels.h"

namespace dl {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Lane layout of v_mfma_f32_16x16x32_bf16 (lane l, n = l % 16, g = l / 16):
// A[n][8g + j] and B[8g + j][n] for j < 8 (8 consecutive K values, one
// 16-byte load from a K-contiguous row), D[4g + i][n] for i < 4.
__device__ __forceinline__ bf16x8 as_bf16x8(const uint4 &v) {
  v4u u = {v.x, v.y, v.z, v.w};
  return __builtin_bit_cast(bf16x8, u);
}
__device__ __forceinline__ f32x4 mfma_bf16(const uint4 &a, const uint4 &b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

__device__ __forceinline__ unsigned pack_bf16(float a, float b) {  // round to nearest even
  f32x2 f = {a, b};
  return __builtin_bit_cast(unsigned, __builtin_convertvector(f, bf16x2));
}
// x = hi + lo as two packed bf16 octets (element j in bits 16j.. of the octet).
__device__ __forceinline__ void split8(const float (&x)[8], uint4 &hi, uint4 &lo) {
  unsigned h[4], l[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const unsigned ua = __float_as_uint(x[2 * j]) & 0xffff0000u;
    const unsigned ub = __float_as_uint(x[2 * j + 1]) & 0xffff0000u;
    h[j] = (ua >> 16) | ub;
    l[j] = pack_bf16(x[2 * j] - __uint_as_float(ua), x[2 * j + 1] - __uint_as_float(ub));
  }
  hi = make_uint4(h[0], h[1], h[2], h[3]);
  lo = make_uint4(l[0], l[1], l[2], l[3]);
}
__device__ __forceinline__ void load8f(const float *p, float (&x)[8]) {
  const float4 u = ld16f(p), v = ld16f(p + 4);
  x[0] = u.x; x[1] = u.y; x[2] = u.z; x[3] = u.w;
  x[4] = v.x; x[5] = v.y; x[6] = v.z; x[7] = v.w;
}

// One wave: acc[c] += A_c (16 x 32 nks) . W^T (32 nks x 16) with bf16 A rows
// at ap[c] and weight rows at wp (both already offset by this lane's row and
// its 8g K position).  U K-steps of loads per batch; the K-steps of the last
// batch beyond nks re-read step nks-1 and multiply zero weights.
template <int NC, int U>
__device__ __forceinline__ void mfma_rows(const uint16_t *wp, const uint16_t *const (&ap)[NC], int nks,
                                          f32x4 (&acc)[NC]) {
  for (int ks = 0; ks < nks; ks += U) {
    uint4 wv[U], av[U][NC];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int k = min(ks + u, nks - 1) * 32;
      wv[u] = ld16(wp + k);
#pragma unroll
      for (int c = 0; c < NC; ++c) av[u][c] = ld16(ap[c] + k);
    }
    DL_SCHED_FENCE();
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint4 w = zero_unless(ks + u < nks, wv[u]);
#pragma unroll
      for (int c = 0; c < NC; ++c) acc[c] = mfma_bf16(av[u][c], w, acc[c]);
    }
  }
}

template <class Fn>
__device__ __forceinline__ void by_chunks(int nc, Fn fn) {
  switch (nc) {
    case 1: fn(std::integral_constant<int, 1>{}); break;
    case 2: fn(std::integral_constant<int, 2>{}); break;
    case 3: fn(std::integral_constant<int, 3>{}); break;
    default: fn(std::integral_constant<int, 4>{}); break;
  }
}

// ================================================================ launch 1
// NR row tiles x NC 16-token chunks per wave, K split over the waves: per K
// step a wave loads NR weight fragments and NC activation fragments and
// runs NR * NC matrix-core steps, so a workgroup reads as many activation
// bytes as weight bytes (with 16-row tiles per workgroup it read NC times
// more).  U K steps of loads per batch; the K steps of the last batch beyond
// nks re-read step nks-1 and multiply zero weights.
template <int NR, int NC, int U>
__device__ __forceinline__ void mfma_tiles(const uint16_t *const (&wp)[NR], const uint16_t *const (&ap)[NC], int nks,
                                           f32x4 (&acc)[NR][NC]) {
  for (int ks = 0; ks < nks; ks += U) {
    uint4 wv[U][NR], av[U][NC];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int k = min(ks + u, nks - 1) * 32;
#pragma unroll
      for (int r = 0; r < NR; ++r) wv[u][r] = ld16(wp[r] + k);
#pragma unroll
      for (int c = 0; c < NC; ++c) av[u][c] = ld16(ap[c] + k);
    }
    DL_SCHED_FENCE();
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        const uint4 w = zero_unless(ks + u < nks, wv[u][r]);
#pragma unroll
        for (int c = 0; c < NC; ++c) acc[r][c] = mfma_bf16(av[u][c], w, acc[r][c]);
      }
  }
}

constexpr int kPjRowWords = 128 * 8;  // 16-byte words of one wave's relayout rows (128 rows x 128 bytes)

// The same product with the operands loaded into registers as 8 rows x 128
// contiguous bytes per instruction (whole cache lines; 64-element K chunks,
// two matrix-core K steps) and moved into the matrix-core layout through the
// wave's own LDS rows (word c of row R at slot c ^ ((R >> 1) & 7), free of
// bank conflicts).  The next chunk's loads are issued before the current
// chunk is used (two register buffers), so the loads overlap the work.
template <int NR, int NC>
__device__ __forceinline__ void mfma_tiles_reg(const uint16_t *w0, size_t wld, int nw, const uint16_t *a0, size_t ald,
                                               int na, int nks, uint4 *ws, f32x4 (&acc)[NR][NC]) {
  constexpr int NI = (NR + NC) * 2;  // load instructions per chunk (8 rows each)
  const int lane = threadIdx.x & 63, n = lane & 15, g = lane >> 4, lr = lane >> 3, lw = lane & 7;
  const int nch = (nks + 1) >> 1;
  auto load = [&](int j, uint4 (&v)[NI]) {
    j = min(j, nch - 1);  // past the last chunk: reload it (unused), so every load issues
    const int wd = 2 * j + (lw >> 2) < nks ? lw : (lw & 3);  // a K step past the range re-reads step 2j
#pragma unroll
    for (int q = 0; q < NI; ++q) {
      const int R = 8 * q + lr;
      const uint16_t *src = R < NR * 16 ? w0 + (size_t)min(R, nw - 1) * wld + 64 * j + 8 * wd
                                        : a0 + (size_t)min(R - NR * 16, na - 1) * ald + 64 * j + 8 * wd;
      v[q] = ld16(src);
    }
  };
  auto use = [&](int j, const uint4 (&v)[NI]) {
#pragma unroll
    for (int q = 0; q < NI; ++q) {
      const int R = 8 * q + lr;
      ws[R * 8 + (lw ^ ((R >> 1) & 7))] = v[q];
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's rows are written
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      if (2 * j + s2 < nks) {
        uint4 wv[NR], av[NC];
#pragma unroll
        for (int r = 0; r < NR; ++r) {
          const int R = 16 * r + n;
          wv[r] = ws[R * 8 + ((4 * s2 + g) ^ ((R >> 1) & 7))];
        }
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          const int R = NR * 16 + 16 * c + n;
          av[c] = ws[R * 8 + ((4 * s2 + g) ^ ((R >> 1) & 7))];
        }
#pragma unroll
        for (int r = 0; r < NR; ++r)
#pragma unroll
          for (int c = 0; c < NC; ++c) acc[r][c] = mfma_bf16(av[c], wv[r], acc[r][c]);
      }
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);  // the reads are done before the next chunk overwrites the rows
    __builtin_amdgcn_wave_barrier();
  };
  uint4 va[NI], vb[NI];
  load(0, va);
  for (int j = 0; j < nch; j += 2) {
    load(j + 1, vb);
    use(j, va);
    if (j + 1 >= nch) break;
    load(j + 2, va);
    use(j + 1, vb);
  }
}

// Workgroup: kProjRows rows of Wo (blocks < n_wo; K = Do split over the 4
// waves) or of Wqkv (K = H split over qkv_split workgroups x 4 waves).
// red[w][token][row]: wave w's partial sum.
constexpr int kProjRows = 64;
__global__ void __launch_bounds__(kBlock) proj_b(BatchArgs a, int n_wo) {
  // each wave's relayout rows during the main loop, then the per-wave partial sums
  __shared__ __align__(16) uint4 lds_raw[kWavesPerBlock * kPjRowWords];
  float (*red)[kMaxBatch][kProjRows] = reinterpret_cast<float (*)[kMaxBatch][kProjRows]>(lds_raw);
  static_assert(sizeof(float) * kWavesPerBlock * kMaxBatch * kProjRows <= sizeof(uint4) * kWavesPerBlock * kPjRowWords, "red fits");
  const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63, n = lane & 15, g = lane >> 4;
  const int B = a.B;
  const bool wo = (int)blockIdx.x < n_wo;
  int r0, split = 0, nks, ld, nrow;
  const uint16_t *wbase, *abase;
  size_t wld;
  if (wo) {
    r0 = blockIdx.x * kProjRows;
    const int kw = wv * (a.Do / 4) + 8 * g;
    wbase = a.w_o + kw;
    wld = a.Do;
    abase = a.attn + kw;
    ld = a.Do;
    nks = a.Do / 128;
    nrow = a.H;
  } else {
    const int b = blockIdx.x - n_wo, S = a.qkv_split;
    r0 = (b / S) * kProjRows;
    split = b % S;
    const int kq = a.H / (S * kWavesPerBlock);
    const int kw = split * (a.H / S) + wv * kq + 8 * g;
    wbase = a.w_qkv + kw;
    wld = a.H;
    abase = a.x + kw;
    ld = a.H;
    nks = kq / 32;
    nrow = a.Dq;
  }
  // the residual rows of this workgroup's tokens, requested before the
  // weights so the epilogue does not wait on a load per token
  constexpr int TPW = kMaxBatch / kWavesPerBlock;  // tokens per wave in the epilogue
  float rin[TPW];
  if (wo) {
#pragma unroll
    for (int j = 0; j < TPW; ++j) rin[j] = a.resid_in[(size_t)min(wv + kWavesPerBlock * j, B - 1) * a.H + r0 + lane];
  }
  constexpr int NR = kProjRows / 16;
  by_chunks((B + 15) >> 4, [&](auto ncc) {
    constexpr int NC = decltype(ncc)::value;
    f32x4 acc[NR][NC];
#pragma unroll
    for (int r = 0; r < NR; ++r)
#pragma unroll
      for (int c = 0; c < NC; ++c) acc[r][c] = f32x4{0.f, 0.f, 0.f, 0.f};
    // rows r0.. of the weights and tokens 0.. from this wave's K start
    mfma_tiles_reg<NR, NC>(wbase - 8 * g + (size_t)r0 * wld, wld, nrow - r0, abase - 8 * g, (size_t)ld, B, nks,
                           lds_raw + wv * kPjRowWords, acc);
    __syncthreads();  // the partial sums below overwrite other waves' staging buffers
#pragma unroll
    for (int r = 0; r < NR; ++r)
#pragma unroll
      for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int i = 0; i < 4; ++i) red[wv][16 * c + 4 * g + i][16 * r + n] = acc[r][c][i];
  });
  __syncthreads();
  if (wo) {
    // wave wv takes token 4j + wv with its 64 rows in the lanes
    const int i = r0 + lane;
    const float gi = bf16_lo(a.gain[i]);
#pragma unroll
    for (int j = 0; j < TPW; ++j) {
      const int t = wv + kWavesPerBlock * j;
      if (t < B) {
        const float s = ((red[0][t][lane] + red[1][t][lane]) + red[2][t][lane]) + red[3][t][lane];
        const size_t o = (size_t)t * a.H + i;
        const float r1 = rin[j] + s;
        a.resid_out[o] = r1;
        a.hg[o] = gi * r1;
        const float sq = wave_sum(r1 * r1);
        if (lane == 0) a.ss_part[(size_t)blockIdx.x * B + t] = sq;
      }
    }
  } else {
    for (int q = tid; q < B * kProjRows; q += kBlock) {
      const int t = q / kProjRows, nn = q % kProjRows, j = r0 + nn;
      if (j < a.Dq)
        a.qkv_part[((size_t)split * B + t) * a.Dq + j] =
            ((red[0][t][nn] + red[1][t][nn]) + red[2][t][nn]) + red[3][t][nn];
    }
  }
}

// ================================================================ launch 2
// Lane layout of v_mfma_f32_16x16x4_f32: A[n][g], B[g][n], D[4g + i][n].
// The K axis is permuted the same way for both operands so that every lane
// reads 4 consecutive fp32 values: at sub-step s, MFMA K index g stands for
// k = kb + 4g + s.
__global__ void __launch_bounds__(kBlock) router_b(BatchArgs a) {
  constexpr int NT = kBatchRtrExperts / 16;  // expert tiles per workgroup
  // staging: per wave, the 64-element K range of its NT*16 expert rows and
  // up to 64 token rows, 256 bytes per row (16 words); then the partial sums
  constexpr int RW = NT * 16 + kMaxBatch;     // staged rows per wave
  __shared__ __align__(16) uint4 lds_raw[kWavesPerBlock * RW * 16];
  float (*red)[4 * NT * 256] = reinterpret_cast<float (*)[4 * NT * 256]>(lds_raw);  // [wave][chunk][tile][m * 16 + n]
  static_assert(sizeof(float) * kWavesPerBlock * 4 * NT * 256 <= sizeof(uint4) * kWavesPerBlock * RW * 16, "red fits");
  static_assert(kBatchRtrK / kWavesPerBlock == 64, "one 256-byte fp32 segment per row and wave");
  const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63, n = lane & 15, g = lane >> 4;
  const int B = a.B, H = a.H, E = a.E;
  // Workgroups are dealt to the 8 XCDs round-robin by linear id, so ids L,
  // L + 8, ... share one XCD's L2.  Tiles (K chunk ky, expert group ex) are
  // numbered with ex fastest and each XCD takes a contiguous range of them:
  // its workgroups then share a few hg K chunks instead of every XCD reading
  // every chunk.
  const int nb = gridDim.x * gridDim.y, lin = blockIdx.y * gridDim.x + blockIdx.x;
  const int tile = nb % 8 == 0 ? (lin % 8) * (nb / 8) + lin / 8 : lin;
  const int e0 = (tile % gridDim.x) * kBatchRtrExperts, ky = tile / gridDim.x;
  const int kb0 = ky * kBatchRtrK + wv * (kBatchRtrK / kWavesPerBlock);  // this wave's K start
  uint4 *buf = lds_raw + wv * RW * 16;
  by_chunks((B + 15) >> 4, [&](auto ncc) {
    constexpr int NC = decltype(ncc)::value;
    // rows R < NT*16 are experts e0 + R, the rest tokens; each load
    // instruction covers 4 rows x 256 contiguous bytes (word c of row R at
    // slot c ^ (R & 15), so the operand reads below are conflict-free)
    constexpr int NI = (NT * 16 + NC * 16) / 4;
#pragma unroll
    for (int q = 0; q < NI; ++q) {
      const int R = 4 * q + (lane >> 4), p = lane & 15, c = p ^ (R & 15);
      const float *src = R < NT * 16 ? a.w_router + (size_t)min(e0 + R, E - 1) * H + kb0 + 4 * c
                                     : a.hg + (size_t)min(R - NT * 16, B - 1) * H + kb0 + 4 * c;
      __builtin_amdgcn_global_load_lds((const void *)src, (__attribute__((address_space(3))) void *)(buf + 64 * q), 16, 0, 0);
    }
    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): the rows are in LDS
    // lane (n, g) at step it takes word 4 it + g: K = 16 it + 4 g .. + 3
    float4 bw[4][NT], av[4][NC];
#pragma unroll
    for (int it = 0; it < 4; ++it) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const int R = 16 * nt + n;
        bw[it][nt] = __builtin_bit_cast(float4, buf[R * 16 + ((4 * it + g) ^ (R & 15))]);
      }
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const int R = NT * 16 + 16 * c + n;
        av[it][c] = __builtin_bit_cast(float4, buf[R * 16 + ((4 * it + g) ^ (R & 15))]);
      }
    }
    f32x4 acc[NC][NT];
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) acc[c][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int it = 0; it < 4; ++it)
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const float x[4] = {av[it][c].x, av[it][c].y, av[it][c].z, av[it][c].w};
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const float w4[4] = {bw[it][nt].x, bw[it][nt].y, bw[it][nt].z, bw[it][nt].w};
#pragma unroll
          for (int s = 0; s < 4; ++s) acc[c][nt] = __builtin_amdgcn_mfma_f32_16x16x4f32(x[s], w4[s], acc[c][nt], 0, 0, 0);
        }
      }
    __syncthreads();  // the partial sums below overlay other waves' staging rows
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i) red[wv][(c * NT + nt) * 256 + (4 * g + i) * 16 + n] = acc[c][nt][i];
  });
  __syncthreads();
  for (int q = tid; q < B * kBatchRtrExperts; q += kBlock) {
    const int t = q / kBatchRtrExperts, el = q % kBatchRtrExperts;
    const int idx = ((t >> 4) * NT + (el >> 4)) * 256 + (t & 15) * 16 + (el & 15);
    if (e0 + el < E)
      a.rlog_part[((size_t)ky * B + t) * E + e0 + el] =
          ((red[0][idx] + red[1][idx]) + red[2][idx]) + red[3][idx];
  }
  // qkv = sum of the K-split partials, spread over the grid
  const int nblk = gridDim.x * gridDim.y, bl = blockIdx.y * gridDim.x + blockIdx.x;
  const size_t nq = (size_t)B * a.Dq, plane = nq;
  for (size_t q = (size_t)bl * kBlock + tid; q < nq; q += (size_t)nblk * kBlock) {
    const float *p = a.qkv_part + q;
    float pv[kBatchQkvSplit];  // every split's load issued before the sum
#pragma unroll
    for (int sp = 0; sp < kBatchQkvSplit; ++sp) pv[sp] = p[min(sp, a.qkv_split - 1) * plane];
    float v = pv[0];
#pragma unroll
    for (int sp = 1; sp < kBatchQkvSplit; ++sp)
      if (sp < a.qkv_split) v += pv[sp];
    a.qkv[q] = v;
  }
}

// Exclusive prefix sums of two per-thread counts over the workgroup (kBlock
// threads), with the totals: a scan inside each wave, then the wave totals
// from LDS (two barriers instead of one pair per doubling step).
__device__ __forceinline__ void block_excl_scan2(int x, int y, int &px, int &py, int &tx, int &ty, int *sx, int *sy) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  int ix = x, iy = y;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const int vx = __shfl_up(ix, d, kWave), vy = __shfl_up(iy, d, kWave);
    if (lane >= d) {
      ix += vx;
      iy += vy;
    }
  }
  __syncthreads();  // earlier readers of sx / sy are done
  if (lane == kWave - 1) {
    sx[wv] = ix;
    sy[wv] = iy;
  }
  __syncthreads();
  int ox = 0, oy = 0;
  tx = 0;
  ty = 0;
#pragma unroll
  for (int w = 0; w < kWavesPerBlock; ++w) {
    const int wx = sx[w], wy = sy[w];
    if (w < wv) {
      ox += wx;
      oy += wy;
    }
    tx += wx;
    ty += wy;
  }
  px = ox + ix - x;
  py = oy + iy - y;
}

// ================================================================ launch 3
__global__ void __launch_bounds__(kBlock) topk_b(BatchArgs a, int n_ow, int n_rk) {
  __shared__ float lg[kMaxExperts];
  __shared__ float wred[kWavesPerBlock];
  __shared__ int cnt[kMaxExperts], off[kMaxExperts];
  __shared__ unsigned msk[kMaxExperts][2];
  __shared__ int sa[kBlock], sc[kBlock];
  __shared__ int slot_nch[kMaxExperts];
  __shared__ int s_pe[kMaxBatch * kMaxTopK];   // the last workgroup: every pick's expert
  __shared__ float s_pw[kMaxBatch * kMaxTopK]; // and weight
  __shared__ int last_flag;
  __shared__ unsigned s_tk_key[kWave];  // split top-k: each wave's picks
  __shared__ int s_tk_idx[kWave];
  const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63;
  const int B = a.B, H = a.H, E = a.E, K = a.K, t = blockIdx.x;
  // every load of the token's hg row is requested together with the norm's
  // partial sums (one round trip instead of one per loop pass)
  constexpr int HJ = 16384 / (kBlock * 8);  // 8-element chunks per thread (H <= 16384)
  float4 hx[HJ][2];
#pragma unroll
  for (int j = 0; j < HJ; ++j) {
    const int i = tid * 8 + kBlock * 8 * j;
    if (i < H) {
      hx[j][0] = ld16f(a.hg + (size_t)t * H + i);
      hx[j][1] = ld16f(a.hg + (size_t)t * H + i + 4);
    }
  }
  // the router partial sums of this thread's experts (e = tid, tid + kBlock)
  // are requested in the same round trip: the logits need 1/rms only at the end
  constexpr int PRE = 32;  // K chunks preloaded per expert
  const bool pre = n_rk <= PRE && E <= 2 * kBlock;
  const size_t lstride = (size_t)B * E;
  float pv[2][PRE];
  if (pre) {
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      const float *p = a.rlog_part + (size_t)t * E + min(tid + kBlock * x, E - 1);
#pragma unroll
      for (int j = 0; j < PRE; ++j) pv[x][j] = p[min(j, n_rk - 1) * lstride];
    }
  }
  // 1/rms from the out-projection workgroups' partial sums
  float ss = 0.f;
  for (int q = tid; q < n_ow; q += kBlock) ss += a.ss_part[(size_t)q * B + t];
  ss = wave_sum(ss);
  if (lane == 0) wred[wv] = ss;
  __syncthreads();
  const float inv = 1.0f / sqrtf(((wred[0] + wred[1]) + (wred[2] + wred[3])) / (float)H + a.eps);
  // h = hg / rms: fp32 copy, optional output, bf16 hi/lo planes
#pragma unroll
  for (int j = 0; j < HJ; ++j) {
    const int i = tid * 8 + kBlock * 8 * j;
    if (i >= H) break;
    const size_t o = (size_t)t * H + i;
    float x[8] = {hx[j][0].x, hx[j][0].y, hx[j][0].z, hx[j][0].w, hx[j][1].x, hx[j][1].y, hx[j][1].z, hx[j][1].w};
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) x[jj] *= inv;
    const float4 u = make_float4(x[0], x[1], x[2], x[3]), v = make_float4(x[4], x[5], x[6], x[7]);
    *reinterpret_cast<float4 *>(a.hn + o) = u;
    *reinterpret_cast<float4 *>(a.hn + o + 4) = v;
    if (a.h_out) {
      *reinterpret_cast<float4 *>(a.h_out + o) = u;
      *reinterpret_cast<float4 *>(a.h_out + o + 4) = v;
    }
    uint4 hi, lo;
    split8(x, hi, lo);
    *reinterpret_cast<uint4 *>(a.hp + o) = hi;
    *reinterpret_cast<uint4 *>(a.hp + (size_t)B * H + o) = lo;
  }
  // logits: K chunks summed in ascending order, then scaled
  if (pre) {
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      const int e = tid + kBlock * x;
      if (e < E) {
        float d = 0.f;
#pragma unroll
        for (int j = 0; j < PRE; ++j) d += j < n_rk ? pv[x][j] : 0.f;
        const float l = d * inv;
        lg[e] = l;
        if (a.logits_out) a.logits_out[(size_t)t * E + e] = l;
      }
    }
  }
  for (int e = pre ? E : tid; e < E; e += kBlock) {
    float d = 0.f;
    const float *p = a.rlog_part + (size_t)t * E + e;
    const size_t stride = (size_t)B * E;
    for (int ky0 = 0; ky0 < n_rk; ky0 += 32) {  // 32 independent loads per batch
      float v[32];
#pragma unroll
      for (int j = 0; j < 32; ++j) v[j] = p[min(ky0 + j, n_rk - 1) * stride];
#pragma unroll
      for (int j = 0; j < 32; ++j) d += ky0 + j < n_rk ? v[j] : 0.f;
    }
    const float l = d * inv;
    lg[e] = l;
    if (a.logits_out) a.logits_out[(size_t)t * E + e] = l;
  }
  __syncthreads();
  // The token's candidates over nwk waves, two 64-expert blocks each: every
  // wave takes its k largest (the lowest lane of the first block holding the
  // maximum has the lowest id, so equal logits cost nothing), then wave 0
  // merges the lists, concatenated in expert-id order, in k more rounds.
  const int nwk = (E + 2 * kWave - 1) / (2 * kWave);
  if (nwk <= kWavesPerBlock && nwk * K <= kWave) {
    unsigned pk;
    int pi;
    if (wv < nwk) {
      unsigned key[2];
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const int e = 2 * kWave * wv + kWave * c + lane;
        key[c] = e < E ? rank_bits(lg[e]) : 0u;
      }
      wave_topk_blocks<2>(key, 2 * kWave * wv, K, pk, pi);
      if (lane < K) {
        s_tk_key[wv * K + lane] = pk;
        s_tk_idx[wv * K + lane] = pi;
      }
    }
    __syncthreads();
    if (wv == 0) {
      wave_topk_merge(lane < nwk * K ? s_tk_key[lane] : 0u, lane < nwk * K ? s_tk_idx[lane] : 0, K, pk, pi);
      const float wgt = pick_weights(unrank_bits(pk), K);
      if (lane < K) {  // written through: the last workgroup reads them back
        __hip_atomic_store(a.topk_idx + (size_t)t * K + lane, pi, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(a.topk_w + (size_t)t * K + lane, wgt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  } else if (wv == 0) {  // lane holds experts lane, lane + 64, ... (as many as E needs)
    int my_idx;
    float my_l;
    auto pick = [&](auto ncc) {
      constexpr int NCAND = decltype(ncc)::value;
      float lv[NCAND];
#pragma unroll
      for (int c = 0; c < NCAND; ++c) {
        const int e = lane + 64 * c;
        lv[c] = e < E ? lg[e] : 0.f;
      }
      wave_topk<NCAND>(lv, E, K, my_idx, my_l);
    };
    if (E <= 128) pick(std::integral_constant<int, 2>{});
    else if (E <= 256) pick(std::integral_constant<int, 4>{});
    else if (E <= 384) pick(std::integral_constant<int, 6>{});
    else if (E <= 512) pick(std::integral_constant<int, 8>{});
    else pick(std::integral_constant<int, kMaxExperts / kWave>{});
    const float wgt = pick_weights(my_l, K);
    if (lane < K) {  // written through: the last workgroup reads them back
      __hip_atomic_store(a.topk_idx + (size_t)t * K + lane, my_idx, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(a.topk_w + (size_t)t * K + lane, wgt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  if (!arrive_last_wt(a.counter, B, &last_flag)) return;

  // ---- the last workgroup: per-expert token lists ----
  for (int q = tid; q < E; q += kBlock) {
    cnt[q] = 0;
    msk[q][0] = msk[q][1] = 0u;
  }
  __syncthreads();
  const int P = B * K;
  for (int i = tid; i < P; i += kBlock) {  // each pick read once, kept in LDS
    const int e = __hip_atomic_load(a.topk_idx + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT), tt = i / K;
    const float wgt = __hip_atomic_load(a.topk_w + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_pe[i] = e;
    s_pw[i] = wgt;
    atomicAdd(&cnt[e], 1);
    atomicOr(&msk[e][tt >> 5], 1u << (tt & 31));
  }
  __syncthreads();
  // exclusive scans over experts: active-slot index and pair offset
  const int seg = (E + kBlock - 1) / kBlock;
  const int q0 = tid * seg, q1 = min(E, q0 + seg);
  int la = 0, lc = 0;
  for (int q = q0; q < q1; ++q) { la += cnt[q] > 0; lc += cnt[q]; }
  int pa, pc, n_act, n_pairs;
  block_excl_scan2(la, lc, pa, pc, n_act, n_pairs, sa, sc);
  for (int q = q0; q < q1; ++q) {
    const int c = cnt[q];
    off[q] = pc;
    if (c > 0) {
      a.act_exp[pa] = q;
      a.act_cnt[pa] = c;
      a.act_off[pa] = pc;
      // gate/up work per slot: 16-token chunks on the matrix cores, else one VALU entry
      slot_nch[pa] = c >= kBatchMfmaMin ? (c + 15) >> 4 : 0;
      ++pa;
      pc += c;
    }
  }
  if (tid == kBlock - 1) *a.n_active = n_act;
  __syncthreads();
  // gate/up work lists: matrix-core entries (slot, 16-token chunk), then VALU
  // entries (slot, all of its fewer than 16 tokens); slots ascending in each
  {
    const int seg2 = (n_act + kBlock - 1) / kBlock;
    const int s0 = tid * seg2, s1 = min(n_act, s0 + seg2);
    int lm = 0, lv = 0;
    for (int q = s0; q < s1; ++q) {
      lm += slot_nch[q];
      lv += slot_nch[q] == 0;
    }
    int pm, pv, n_qm, n_qv;
    block_excl_scan2(lm, lv, pm, pv, n_qm, n_qv, sa, sc);
    pv += n_qm;
    for (int q = s0; q < s1; ++q) {
      for (int c = 0; c < slot_nch[q]; ++c) a.gu_q[pm++] = q | (c << 16);
      if (slot_nch[q] == 0) a.gu_q[pv++] = q;
    }
    if (tid == kBlock - 1) {
      a.n_q[0] = n_qm;
      a.n_q[1] = n_qv;
    }
  }
  __syncthreads();
  // a pair's place inside its expert = number of lower tokens with that expert
  for (int i = tid; i < P; i += kBlock) {
    const int e = s_pe[i], tt = i / K;
    const unsigned m0 = msk[e][0], m1 = msk[e][1];
    const int r = tt < 32 ? __popc(m0 & ((1u << tt) - 1u)) : __popc(m0) + __popc(m1 & ((1u << (tt - 32)) - 1u));
    const int pos = off[e] + r;
    a.pair_tok[pos] = tt;
    a.pair_w[pos] = s_pw[i];
  }
}

// ================================================================ launch 4
struct GuItem {
  const uint16_t *w1, *w3;  // first of the item's 16 rows, row stride H
  const int *toks;          // token of row m (nullptr: tok0 + m)
  int tok0;
  float *out;               // row m of the output at out + m * ld, 16 columns
  int ld, cnt;              // cnt <= 16 rows on the matrix cores, < 16 on the VALU
  __device__ int tok(int m) const { return toks ? toks[m] : tok0 + m; }
};

// Fewer than 16 tokens: wave w takes rows 4w .. 4w+3 of the item, one
// (W1 row, W3 row) pair at a time over the full K, up to 8 tokens per pass.
__device__ void gateup_valu(const BatchArgs &a, const GuItem &it) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int H = a.H;
  for (int t0 = 0; t0 < it.cnt; t0 += 8) {
    const int nt = min(8, it.cnt - t0);
    auto pass = [&](auto ntc) {
      constexpr int NT = decltype(ntc)::value;
      constexpr int CPB = NT <= 2 ? 4 : NT <= 4 ? 2 : 1;
      HgGather<NT> act;
      act.base = a.hn;
      act.ld = H;
#pragma unroll
      for (int t = 0; t < NT; ++t) act.tok[t] = it.tok(t0 + min(t, nt - 1));
      for (int r = 0; r < 4; ++r) {
        const int f = 4 * wv + r;
        const uint16_t *w[2] = {it.w1 + (size_t)f * H, it.w3 + (size_t)f * H};
        float o[2][NT];
        wave_rows_dot<2, NT, CPB>(w, 0, H / 8, act, o);
#pragma unroll
        for (int t = 0; t < NT; ++t)
          if (lane == t && t < nt) it.out[(size_t)(t0 + t) * it.ld + f] = silu_mul(o[0][t], o[1][t]);
      }
    };
    if (nt == 1) pass(std::integral_constant<int, 1>{});
    else if (nt == 2) pass(std::integral_constant<int, 2>{});
    else if (nt <= 4) pass(std::integral_constant<int, 4>{});
    else pass(std::integral_constant<int, 8>{});
  }
}

// Matrix-core units.  A group is 16 NTL rows (NTL <= 4) of W1 and the same
// rows of W3 applied to one 16-token chunk: a chunk of a routed expert with
// 16 or more tokens, or of the shared expert when B >= 16.  A unit is one
// group over kGuKc K steps of 32 (448 K elements at H = 7168; a group has
// ceil(H / (32 kGuKc)) units, its K chunks).  The workgroup stages the
// chunk's activations for the unit's K range (bf16 hi and lo planes of h)
// in LDS with contiguous loads; wave w < NTL then streams the 16 rows of
// tile w of W1 and of W3, 7 K steps (448 bytes of each row) per load batch,
// taking its activation fragments from LDS.  The sums go to the group's
// slot for that K chunk, written through to the device coherence point; the
// last unit of the group to arrive adds the slots in K-chunk order (so the
// result does not depend on arrival order) and writes silu(u) * v.
// VALU units.  (expert, 16-row tile) of experts with fewer than 16 tokens,
// and of the shared expert below 16 tokens, after the matrix-core units.
constexpr int kGuPad = 8;                  // bf16 elements of padding per LDS row
constexpr int kGuLd = 32 * kGuKc + kGuPad; // LDS row of one staged token
constexpr int kGuLds = 2 * 16 * kGuLd * 2; // bytes: [hi | lo][16 tokens][kGuLd]
constexpr unsigned kGuSc1 = 16;            // cache policy: coherent at agent scope

struct GuUnit {
  const uint16_t *w1, *w3;  // row 0 of the group, row stride H
  float *out;               // output row m at out + m * ld, columns [0, 16 NTL)
  float *slots;             // the group's slots, kGuSlotFloatsR floats each
  unsigned *arrivals;       // the group's arrival counter
  int ld, cnt, k0, k1, kc, nck, ntl, group;
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t gu_rsrc(const float *p, int floats) {
  return __builtin_amdgcn_make_buffer_rsrc((void *)p, 0, floats * 4, 0x00020000);
}

// One matrix-core unit: sums over its K chunk into its slot, as
// [W1 | W3][tile][row][token] (a lane's 4 tokens are contiguous).
// Weights are loaded by pairs of K steps, 8 rows x 128 contiguous bytes per
// instruction (whole cache lines), and moved into the matrix-core layout
// through the wave's own 4 KB of LDS (ws): word c of row r of a pair sits at
// slot c ^ ((r >> 1) & 7), so writes and reads are free of bank conflicts.
constexpr int kGuPairs = 4;  // K-step pairs per load batch
template <int NTL>
__device__ void gu_unit(const BatchArgs &a, const GuUnit &s, const uint16_t *lds, uint4 *ws) {
  const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63, n = lane & 15, g = lane >> 4;
  if (wv >= NTL) return;
  const int H = a.H, kb = 32 * s.k0, nks = s.k1 - s.k0, npair = (nks + 1) >> 1;
  // load lane: rows 8h + lane / 8 of the tile, word lane % 8 of a pair
  const int lr = lane >> 3, lw = lane & 7;
  const uint16_t *q1[2], *q3[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    q1[h] = s.w1 + (size_t)(16 * wv + 8 * h + lr) * H + kb;
    q3[h] = s.w3 + (size_t)(16 * wv + 8 * h + lr) * H + kb;
  }
  const uint16_t *lh = lds + n * kGuLd + 8 * g, *ll = lh + 16 * kGuLd;
  f32x4 acc1 = {0.f, 0.f, 0.f, 0.f}, acc3 = acc1;
  for (int p0 = 0; p0 < npair; p0 += kGuPairs) {
    uint4 w1v[kGuPairs][2], w3v[kGuPairs][2];
#pragma unroll
    for (int pp = 0; pp < kGuPairs; ++pp) {
      const int pr = min(p0 + pp, npair - 1);
      // a second K step past the unit re-reads the first (its product is skipped)
      const int wd = 2 * pr + (lw >> 2) < nks ? lw : (lw & 3);
      const int k = 64 * pr + 8 * wd;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        w1v[pp][h] = ld16(q1[h] + k);
        w3v[pp][h] = ld16(q3[h] + k);
      }
    }
    DL_SCHED_FENCE();
#pragma unroll
    for (int pp = 0; pp < kGuPairs; ++pp) {
      const int pr = p0 + pp;
      if (pr >= npair) break;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int r = 8 * h + lr, sl = r * 8 + (lw ^ ((r >> 1) & 7));
        ws[sl] = w1v[pp][h];
        ws[128 + sl] = w3v[pp][h];
      }
      __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's rows are written
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const int ks = 2 * pr + s2;
        if (ks < nks) {
          const int sl = n * 8 + ((4 * s2 + g) ^ ((n >> 1) & 7));
          const uint4 b1 = ws[sl], b3 = ws[128 + sl];
          const uint4 hv = *reinterpret_cast<const uint4 *>(lh + 32 * ks);
          const uint4 lv = *reinterpret_cast<const uint4 *>(ll + 32 * ks);
          acc1 = mfma_bf16(hv, b1, acc1);
          acc3 = mfma_bf16(hv, b3, acc3);
          acc1 = mfma_bf16(lv, b1, acc1);
          acc3 = mfma_bf16(lv, b3, acc3);
        }
      }
      __builtin_amdgcn_wave_barrier();
    }
  }
  const __amdgpu_buffer_rsrc_t r = gu_rsrc(s.slots, s.nck * kGuSlotFloatsR);
  const int base = s.kc * kGuSlotFloatsR + (wv * 16 + n) * 16 + 4 * g;
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u, acc1), r, base * 4, 0, kGuSc1);
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u, acc3), r, (base + NTL * 256) * 4, 0, kGuSc1);
}

// The group's last unit: u and v summed over the K-chunk slots in order.
template <int NTL>
__device__ void gu_combine(const GuUnit &s) {
  constexpr int ROWS = 16 * NTL;
  const int q = threadIdx.x;
  if (q >= ROWS * 4) return;
  const int r = q % ROWS, mq = q / ROWS, t = r >> 4, nn = r & 15;
  const __amdgpu_buffer_rsrc_t rs = gu_rsrc(s.slots, s.nck * kGuSlotFloatsR);
  const int i1 = ((0 * NTL + t) * 16 + nn) * 16 + 4 * mq, i3 = ((NTL + t) * 16 + nn) * 16 + 4 * mq;
  f32x4 u = {0.f, 0.f, 0.f, 0.f}, v = u;
  for (int s0 = 0; s0 < s.nck; s0 += 8) {
    f32x4 pu[8], pv[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int o = min(s0 + j, s.nck - 1) * kGuSlotFloatsR;
      pu[j] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, (o + i1) * 4, 0, kGuSc1));
      pv[j] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, (o + i3) * 4, 0, kGuSc1));
    }
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (s0 + j < s.nck) {
        u += pu[j];
        v += pv[j];
      }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = 4 * mq + i;
    if (m < s.cnt) s.out[(size_t)m * s.ld + r] = silu_mul(u[i], v[i]);
  }
}

// The staged activations of one unit: 16-byte words of [hi | lo][token][K].
constexpr int kGuStW = (2 * 16 * (32 * kGuKc / 8) + kBlock - 1) / kBlock;  // words per thread

__device__ __forceinline__ int gu_token(const int *toks, int tok0, int m, int cnt) {
  m = min(m, cnt - 1);
  return toks ? toks[m] : tok0 + m;
}

__device__ __forceinline__ void gu_stage_load(const BatchArgs &a, const int *tok_l, const GuUnit &s,
                                              uint4 (&st)[kGuStW]) {
  const int kbeg = 32 * s.k0, wpr = 4 * (s.k1 - s.k0), nw = 32 * wpr;
  const size_t plane = (size_t)a.B * a.H;
#pragma unroll
  for (int j = 0; j < kGuStW; ++j) {
    const int w = min((int)threadIdx.x + kBlock * j, nw - 1);
    const int pl = w / (16 * wpr), m = (w / wpr) & 15, c = w % wpr;
    st[j] = ld16(a.hp + pl * plane + (size_t)tok_l[m] * a.H + kbeg + 8 * c);
  }
}

__device__ __forceinline__ void gu_stage_store(const uint4 (&st)[kGuStW], const GuUnit &s, uint16_t *lds) {
  const int wpr = 4 * (s.k1 - s.k0), nw = 32 * wpr;
#pragma unroll
  for (int j = 0; j < kGuStW; ++j) {
    const int w = (int)threadIdx.x + kBlock * j;
    if (w < nw) {
      const int pl = w / (16 * wpr), m = (w / wpr) & 15, c = w % wpr;
      *reinterpret_cast<uint4 *>(lds + (pl * 16 + m) * kGuLd + 8 * c) = st[j];
    }
  }
}

struct GuGeom {
  int NK, NCK, F, Fs, B, rg_r, ngr, rg_s, ng_r, nch_s;
};

// Unit u: its group's weights, output, slots and tokens (toks[m], or tok0 + m).
__device__ __forceinline__ void gu_meta(const BatchArgs &a, const GuGeom &q, int u, GuUnit &s, const int *&toks,
                                        int &tok0) {
  const int gi = u / q.NCK, H = a.H;
  s.group = gi;
  s.nck = q.NCK;
  if (gi < q.ng_r) {
    const int e = gi / q.ngr, r0 = (gi % q.ngr) * q.rg_r;
    const int qe = a.gu_q[e], slot = qe & 0xffff, c0 = 16 * (qe >> 16);
    const int ex = a.act_exp[slot], off = a.act_off[slot] + c0;
    s.w1 = a.w1 + ((size_t)ex * q.F + r0) * H;
    s.w3 = a.w3 + ((size_t)ex * q.F + r0) * H;
    s.cnt = min(16, a.act_cnt[slot] - c0);
    s.out = a.act + (size_t)off * q.F + r0;
    s.ld = q.F;
    s.ntl = q.rg_r >> 4;
    s.slots = a.gu_part + (size_t)gi * q.NCK * kGuSlotFloatsR;
    s.arrivals = a.gu_cnt + gi;
    toks = a.pair_tok + off;
    tok0 = 0;
  } else {
    const int gs = gi - q.ng_r, r0 = (gs / q.nch_s) * q.rg_s, c = gs % q.nch_s;
    s.w1 = a.s1 + (size_t)r0 * H;
    s.w3 = a.s3 + (size_t)r0 * H;
    s.cnt = min(16, q.B - 16 * c);
    s.out = a.act_s + (size_t)(16 * c) * q.Fs + r0;
    s.ld = q.Fs;
    s.ntl = q.rg_s >> 4;
    s.slots = a.gu_part_s + (size_t)gs * q.NCK * kGuSlotFloatsR;
    s.arrivals = a.gu_cnt_s + gs;
    toks = nullptr;
    tok0 = 16 * c;
  }
}

__device__ __forceinline__ void gu_chunk(GuUnit &s, int u, int NK) {
  s.kc = u % s.nck;
  s.k0 = s.kc * kGuKc;
  s.k1 = min(NK, s.k0 + kGuKc);
}

// Matrix-core units laid end to end (group by group, K chunks in order) are
// cut into one contiguous run per workgroup (two workgroups per CU), so
// consecutive units of a workgroup mostly share a group and its tokens.
// While a unit streams its weights, the next unit's activations are loaded
// into registers and then written to the other LDS buffer, so staging does
// not stall the weight stream.  VALU units are dealt round-robin after.
__device__ void dn_plan_runs(const BatchArgs &a, int G_gu, int *s_pre, int *s_wsum);

__global__ void __launch_bounds__(kBlock, 2) gateup_b(BatchArgs a) {
  __shared__ __align__(16) uint16_t lds[2][kGuLds / 2];
  __shared__ __align__(16) uint4 gws[kWavesPerBlock][256];  // each wave's weight pair rows (W1 | W3)
  __shared__ int tok_l[2][16];
  __shared__ int s_flag, s_first;
  __shared__ int s_wsum[kWavesPerBlock];
  const int tid = threadIdx.x;
  const int n_qm = a.n_q[0], n_qv = a.n_q[1];
  GuGeom q;
  q.B = a.B;
  q.F = a.F;
  q.Fs = a.Fs;
  q.NK = a.H >> 5;
  q.NCK = (q.NK + kGuKc - 1) / kGuKc;
  const bool s_mfma = q.Fs > 0 && q.B >= kBatchMfmaMin;
  q.nch_s = s_mfma ? (q.B + 15) >> 4 : 0;
  q.rg_r = min(kBatchGuRows, q.F);
  q.ngr = q.F / q.rg_r;
  q.rg_s = q.Fs > 0 ? min(kBatchGuRows, q.Fs) : 16;
  q.ng_r = n_qm * q.ngr;
  const int ng = q.ng_r + q.nch_s * (q.Fs / q.rg_s);
  const int n_mfma = ng * q.NCK;
  const int G = gridDim.x, w = blockIdx.x;
  // workgroups w and w + G/2 are dispatched to the same CU: give them
  // neighbouring runs, so that every CU holds the same number of units
  const int half = G >> 1, r = (G & 1) ? w : 2 * (w % half) + w / half;
  const int ub = (int)((long)r * n_mfma / G), ue = (int)((long)(r + 1) * n_mfma / G);
  if (ub < ue) {
    GuUnit cur;
    const int *toks;
    int tok0;
    gu_meta(a, q, ub, cur, toks, tok0);
    gu_chunk(cur, ub, q.NK);
    if (tid < 16) tok_l[0][tid] = gu_token(toks, tok0, tid, cur.cnt);
    __syncthreads();
    {
      uint4 st[kGuStW];
      gu_stage_load(a, tok_l[0], cur, st);
      gu_stage_store(st, cur, lds[0]);
    }
    __syncthreads();
    int b = 0;
    for (int u = ub; u < ue; ++u) {
      const bool more = u + 1 < ue;
      GuUnit nx = cur;
      if (more) {
        if ((u + 1) % q.NCK == 0) {  // the next unit starts a new group
          gu_meta(a, q, u + 1, nx, toks, tok0);
          if (tid < 16) tok_l[b ^ 1][tid] = gu_token(toks, tok0, tid, nx.cnt);
        } else if (tid < 16) {
          tok_l[b ^ 1][tid] = tok_l[b][tid];
        }
        gu_chunk(nx, u + 1, q.NK);
      }
      __syncthreads();
      uint4 st[kGuStW];
      if (more) gu_stage_load(a, tok_l[b ^ 1], nx, st);
      asm volatile("" ::: "memory");  // issue the staging loads ahead of the weight stream
      if (cur.ntl == 4) gu_unit<4>(a, cur, lds[b], gws[tid >> 6]);
      else gu_unit<2>(a, cur, lds[b], gws[tid >> 6]);
      if (more) gu_stage_store(st, nx, lds[b ^ 1]);
      // arrival: this workgroup's slot stores have completed before it is counted
      wt_stores_complete();
      __syncthreads();
      if (tid == 0) {
        const unsigned prev = __hip_atomic_fetch_add(cur.arrivals, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s_flag = prev == (unsigned)q.NCK - 1;
        if (s_flag) __hip_atomic_store(cur.arrivals, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      __syncthreads();
      if (s_flag) {
        if (cur.ntl == 4) gu_combine<4>(cur);
        else gu_combine<2>(cur);
      }
      cur = nx;
      b ^= 1;
    }
  }
  const int n_vr = n_qv * (q.F / 16), n_vs = (q.Fs > 0 && !s_mfma) ? q.Fs / 16 : 0;
  for (int i = (w - (n_mfma > 0 ? n_mfma % G : 0) + G) % G; i < n_vr + n_vs; i += G) {
    GuItem it;
    if (i < n_vr) {
      const int slot = a.gu_q[n_qm + i / (q.F / 16)], tile = i % (q.F / 16);
      const int ex = a.act_exp[slot], off = a.act_off[slot];
      it.w1 = a.w1 + ((size_t)ex * q.F + tile * 16) * a.H;
      it.w3 = a.w3 + ((size_t)ex * q.F + tile * 16) * a.H;
      it.toks = a.pair_tok + off;
      it.tok0 = 0;
      it.out = a.act + (size_t)off * q.F + tile * 16;
      it.ld = q.F;
      it.cnt = a.act_cnt[slot];
    } else {
      const int tile = i - n_vr;
      it.w1 = a.s1 + (size_t)tile * 16 * a.H;
      it.w3 = a.s3 + (size_t)tile * 16 * a.H;
      it.toks = nullptr;
      it.tok0 = 0;
      it.out = a.act_s + tile * 16;
      it.ld = q.Fs;
      it.cnt = q.B;
    }
    gateup_valu(a, it);
  }
  // The first workgroup to finish lays out the down projection's runs (it
  // has the other workgroups' remaining gate/up time to do so); the last
  // re-arms the counter.
  if (tid == 0) {
    const unsigned prev = __hip_atomic_fetch_add(a.gu_done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_first = prev == 0u;
    if (prev == (unsigned)G - 1u) __hip_atomic_store(a.gu_done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  // (the staging area is free once every wave has passed that barrier)
  static_assert(sizeof(int) * (kMaxExperts + 2) <= sizeof(lds), "cost prefix fits the staging area");
  if (s_first) dn_plan_runs(a, G, reinterpret_cast<int *>(&lds[0][0]), s_wsum);
}

// ================================================================ launch 5
// Down projection, y[t, i] = S2[i] . a_s[t] + sum_p w_p W2[e_p, i] . a[p].
// Units = (group of 64 rows of y, entry), an entry being one active expert
// (all its tokens) or the shared expert (every token, weight 1).  The
// units, laid end to end group by group, are cut into one contiguous run
// per workgroup (two per CU; the two on one CU take neighbouring runs).
// For a unit, wave w loads rows 16w .. 16w + 15 of the group from the
// entry's weights (all of F: 8 loads of 16 bytes per lane at F = 256), and
// the workgroup stages each 16-token chunk of the entry's activations in
// LDS once — bf16 hi and lo planes for the matrix cores when the entry has
// 16 or more tokens, fp32 rows for the VALU below that — instead of every
// wave re-reading them.  The next unit's weights are requested right after
// the current chunk's activation loads, so they stream during the compute.
// Results are added into an LDS tile y[token][64 rows] (a wave owns its 16
// rows; within an entry a token occurs once, so no two lanes add into one
// element).  When its run leaves a group, the workgroup writes the tile to
// the group's slot numbered by its place among the group's workgroups
// (written through to the device coherence point) and counts itself; the
// last to arrive adds the slots in slot order into moe_out.
// The units laid end to end (group-major, entries in slot order, the shared
// expert last) are cut into runs of equal cost: a unit costs 1 + its number
// of 16-token chunks (its weights once, then one staged chunk of
// activations each), so the shared expert's units at 64 tokens count 5 and
// a hot expert's 2.  Unit u then belongs to workgroup floor(P(u) Ga / C),
// with P(u) the cost of the units before it and C the total.  When no unit
// costs more than C / Ga, consecutive units differ by at most one workgroup,
// so every workgroup between the first and the last of a group holds some
// of its units; otherwise every unit counts 1.  The run bounds are laid out
// by the first gate/up workgroup to finish, so this launch only reads them.
constexpr int kDnRows = 64;
constexpr int kDnLd = 256 + 8;   // bf16 per LDS row of a staged chunk plane (F <= 256)
constexpr int kDnLdF = 256 + 4;  // fp32 per LDS row of a staged VALU chunk

// Run bounds of the down launch (grid min(G_gu, kDnMaxGrid)), by one
// workgroup: the entries' costs and their exclusive prefix s_pre (a scan
// over the workgroup), then for each run w the first unit u with
// P(u) Ga >= w C: group T / S, entry = the smallest i with s_pre[i] >= T mod S
// (T = ceil(w C / Ga), S a group's cost).
__device__ void dn_plan_runs(const BatchArgs &a, int G_gu, int *s_pre, int *s_wsum) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int B = a.B, n_act = *a.n_active;
  const int ne = n_act + (a.Fs > 0 ? 1 : 0), ng = a.H / kDnRows;
  const long U = (long)ng * ne;
  const int Ga = (int)min((long)min(G_gu, kDnMaxGrid), U);
  if (U == 0) return;
  const bool by_cost = (long)(1 + (B + 15) / 16) * Ga <= U;
  constexpr int EPT = (kMaxExperts + kBlock) / kBlock;
  int cq[EPT], run = 0;
#pragma unroll
  for (int j = 0; j < EPT; ++j)  // every load issued (clamped address) before any is used
    cq[j] = a.act_cnt[min(EPT * tid + j, max(n_act - 1, 0))];
#pragma unroll
  for (int j = 0; j < EPT; ++j) {
    const int q = EPT * tid + j;
    const int cnt = q < n_act ? cq[j] : B;
    cq[j] = q >= ne ? 0 : !by_cost ? 1 : 1 + (cnt + 15) / 16;
    run += cq[j];
  }
  int incl = run;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const int t = __shfl_up(incl, d, kWave);
    if (lane >= d) incl += t;
  }
  if (lane == kWave - 1) s_wsum[wv] = incl;
  __syncthreads();
  int before = incl - run;
  for (int v = 0; v < wv; ++v) before += s_wsum[v];
#pragma unroll
  for (int j = 0; j < EPT; ++j) {
    const int q = EPT * tid + j;
    if (q <= ne) s_pre[q] = before;
    before += cq[j];
  }
  __syncthreads();
  const unsigned long long S = (unsigned)s_pre[ne], C = (unsigned long long)ng * S;
  for (int w = tid; w <= Ga; w += kBlock) {
    const unsigned long long T = ((unsigned long long)w * C + (unsigned long long)(Ga - 1)) / (unsigned long long)Ga;
    const unsigned long long g = T / S, rem = T - g * S;
    int lo = 0, hi = ne;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if ((unsigned long long)s_pre[mid] >= rem) hi = mid;
      else lo = mid + 1;
    }
    a.dn_runs[2 + w] = (int)(g * (unsigned long long)ne) + lo;
  }
  if (tid == 0) {
    a.dn_runs[0] = (int)S;
    a.dn_runs[1] = s_pre[ne - 1];
  }
}

__device__ __forceinline__ int dn_run(int w, int G) {
  const int half = G >> 1;
  return (G & 1) ? w : 2 * (w % half) + w / half;
}

// The wave's 16 rows 16 wv .. 16 wv + 15 of the group, loaded as 4 rows x 256
// contiguous bytes per instruction (whole cache lines): word j = 2q + h of a
// lane holds row 4q + lane / 16, 16-byte word (lane % 16) + 16h of the row.
__device__ __forceinline__ void dn_load_w(const uint16_t *rows, int Fd, uint4 (&w)[8]) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int wpr = Fd >> 3;  // 16-byte words per row
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int r = 16 * wv + 4 * q + (lane >> 4), c = min((lane & 15) + 16 * h, wpr - 1);
      w[2 * q + h] = ld16(rows + (size_t)r * Fd + 8 * c);
    }
}

// From the load layout to the matrix-core layout (lane (n, g) at K step s:
// row n, K 32 s + 8 g) through this wave's LDS rows: word c of row r sits at
// slot c ^ (r & 15), so both the writes and the reads are free of bank
// conflicts.  Only this wave touches its rows, and a wave's LDS operations
// run in order.
__device__ __forceinline__ void dn_relayout(const uint4 (&w)[8], uint4 *ws, uint4 (&wm)[8]) {
  const int lane = threadIdx.x & 63, n = lane & 15, g = lane >> 4;
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int r = 4 * q + (lane >> 4), c = (lane & 15) + 16 * h;
      ws[r * 32 + (c ^ (r & 15))] = w[2 * q + h];
    }
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int st = 0; st < 8; ++st) wm[st] = ws[n * 32 + ((4 * st + g) ^ n)];
}

struct DnSrc {
  const float *act;   // chunk row m at act + m * Fd (m < cnt)
  const int *toks;    // token of row m (nullptr: tok0 + m)
  const float *wts;   // weight of row m (nullptr: 1)
  int tok0, cnt, Fd;
};

// Activation loads of one chunk: 8 consecutive fp32 of row m per octet.
__device__ __forceinline__ void dn_stage_load(const DnSrc &c, float4 (&v)[2][2]) {
  const int opr = c.Fd >> 3, no = 16 * opr;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int o = min((int)threadIdx.x + kBlock * j, no - 1), m = min(o / opr, c.cnt - 1), k = 8 * (o % opr);
    const float *p = c.act + (size_t)m * c.Fd + k;
    v[j][0] = ld16f(p);
    v[j][1] = ld16f(p + 4);
  }
}

__device__ __forceinline__ void dn_stage_store(const DnSrc &c, const float4 (&v)[2][2], bool mfma, uint16_t *stg) {
  const int opr = c.Fd >> 3, no = 16 * opr;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int o = (int)threadIdx.x + kBlock * j;
    if (o < no) {
      const int m = o / opr, k = 8 * (o % opr);
      if (mfma) {
        const float x[8] = {v[j][0].x, v[j][0].y, v[j][0].z, v[j][0].w, v[j][1].x, v[j][1].y, v[j][1].z, v[j][1].w};
        uint4 hi, lo;
        split8(x, hi, lo);
        *reinterpret_cast<uint4 *>(stg + m * kDnLd + k) = hi;
        *reinterpret_cast<uint4 *>(stg + (16 + m) * kDnLd + k) = lo;
      } else {
        float *f = reinterpret_cast<float *>(stg) + m * kDnLdF + k;
        *reinterpret_cast<float4 *>(f) = v[j][0];
        *reinterpret_cast<float4 *>(f + 4) = v[j][1];
      }
    }
  }
}

// One staged chunk (rows m < cnt) against this wave's weights, into the tile.
__device__ __forceinline__ void dn_compute(const DnSrc &c, bool mfma, const uint4 (&w)[8], const uint16_t *stg,
                                           const int *s_tok, const float *s_wt, float *ytile) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, n = lane & 15, g = lane >> 4;
  const int nks = c.Fd >> 5, col = 16 * wv + n;
  if (mfma) {
    const uint16_t *lh = stg + n * kDnLd + 8 * g, *ll = lh + 16 * kDnLd;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 8; ++s)
      if (s < nks) {
        const uint4 hv = *reinterpret_cast<const uint4 *>(lh + 32 * s);
        const uint4 lv = *reinterpret_cast<const uint4 *>(ll + 32 * s);
        acc = mfma_bf16(hv, w[s], acc);
        acc = mfma_bf16(lv, w[s], acc);
      }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = 4 * g + i;
      if (m < c.cnt) ytile[s_tok[m] * kDnRows + col] += s_wt[m] * acc[i];
    }
  } else {
    const float *xf = reinterpret_cast<const float *>(stg) + 8 * g;
    for (int m = 0; m < c.cnt; ++m) {
      float acc = 0.f;
#pragma unroll
      for (int s = 0; s < 8; ++s)
        if (s < nks) {
          float wf[8];
          unpack8(w[s], wf);
          const float4 x0 = *reinterpret_cast<const float4 *>(xf + m * kDnLdF + 32 * s);
          const float4 x1 = *reinterpret_cast<const float4 *>(xf + m * kDnLdF + 32 * s + 4);
          acc = fmaf(wf[0], x0.x, acc);
          acc = fmaf(wf[1], x0.y, acc);
          acc = fmaf(wf[2], x0.z, acc);
          acc = fmaf(wf[3], x0.w, acc);
          acc = fmaf(wf[4], x1.x, acc);
          acc = fmaf(wf[5], x1.y, acc);
          acc = fmaf(wf[6], x1.z, acc);
          acc = fmaf(wf[7], x1.w, acc);
        }
      acc += __shfl_xor(acc, 16, kWave);   // lanes g, g ^ 1
      acc += __shfl_xor(acc, 32, kWave);   // (v0 + v1) + (v2 + v3)
      if (g == 0) ytile[s_tok[m] * kDnRows + col] += s_wt[m] * acc;
    }
  }
}

__global__ void __launch_bounds__(kBlock, 2) down_b(BatchArgs a) {
  __shared__ float ytile[kMaxBatch * kDnRows];
  __shared__ __align__(16) uint16_t stg[2 * 16 * kDnLd];
  __shared__ __align__(16) uint4 wst[kWavesPerBlock][16 * 32];  // each wave's 16 weight rows (512 bytes each)
  __shared__ int s_exp[kMaxExperts], s_cnt[kMaxExperts], s_off[kMaxExperts];
  __shared__ int s_tok[16];
  __shared__ float s_wt[16];
  __shared__ int s_flag;
  const int tid = threadIdx.x;
  const int B = a.B, H = a.H, F = a.F, Fs = a.Fs;
  const int n_act = *a.n_active;
  const int ne = n_act + (Fs > 0 ? 1 : 0), ng = H / kDnRows;
  const long U = (long)ng * ne;
  const int G = gridDim.x, ri = dn_run(blockIdx.x, G);
  const int Ga = (int)min((long)G, U);
  if (U == 0 || ri >= Ga) return;
  // this run's units, a group's cost and its cost before its last entry
  long u = a.dn_runs[2 + ri];
  const long ue = a.dn_runs[3 + ri];
  const unsigned long long S = (unsigned)a.dn_runs[0], P_last = (unsigned)a.dn_runs[1];
  for (int q = tid; q < n_act; q += kBlock) {
    s_exp[q] = a.act_exp[q];
    s_cnt[q] = a.act_cnt[q];
    s_off[q] = a.act_off[q];
  }
  for (int q = tid; q < kMaxBatch * kDnRows; q += kBlock) ytile[q] = 0.f;
  __syncthreads();
  const unsigned long long C = (unsigned long long)ng * S;
  const bool narrow = (C + 1ull) * (unsigned long long)Ga < (1ull << 32);
  // workgroup holding unit cost prefix P: floor(P Ga / C)
  auto run_of = [&](unsigned long long P) -> int {
    const unsigned long long x = P * (unsigned long long)Ga;
    return narrow ? (int)((unsigned)x / (unsigned)C) : (int)(x / C);
  };
  auto rows_of = [&](long u, int &Fd) -> const uint16_t * {
    const int r = (int)(u / ne), i = (int)(u % ne);
    if (i < n_act) {
      Fd = F;
      return a.w2 + ((size_t)s_exp[i] * H + (size_t)r * kDnRows) * F;
    }
    Fd = Fs;
    return a.s2 + (size_t)r * kDnRows * Fs;
  };
  uint4 wc[8], wn[8], wm[8];
  {
    int Fd;
    const uint16_t *rows = rows_of(u, Fd);
    dn_load_w(rows, Fd, wc);
  }
  for (; u < ue; ++u) {
    const int r = (int)(u / ne), i = (int)(u % ne);
    const bool routed = i < n_act;
    DnSrc c;
    c.Fd = routed ? F : Fs;
    const int cnt_all = routed ? s_cnt[i] : B;
    const int off = routed ? s_off[i] : 0;
    const bool mfma = cnt_all >= kBatchMfmaMin;
    for (int c0 = 0; c0 < cnt_all; c0 += 16) {
      c.cnt = min(16, cnt_all - c0);
      c.act = routed ? a.act + (size_t)(off + c0) * F : a.act_s + (size_t)c0 * Fs;
      float4 v[2][2];
      dn_stage_load(c, v);
      int tk = 0;
      float wt = 1.f;
      if (tid < 16) {
        const int m = min(tid, c.cnt - 1);
        tk = routed ? a.pair_tok[off + c0 + m] : c0 + m;
        wt = routed ? a.pair_w[off + c0 + m] : 1.f;
      }
      asm volatile("" ::: "memory");
      if (c0 == 0 && u + 1 < ue) {  // the next unit's weights stream during this one
        int Fd;
        const uint16_t *rows = rows_of(u + 1, Fd);
        dn_load_w(rows, Fd, wn);
      }
      asm volatile("" ::: "memory");
      if (c0 == 0) dn_relayout(wc, wst[threadIdx.x >> 6], wm);
      dn_stage_store(c, v, mfma, stg);
      if (tid < 16) {
        s_tok[tid] = tk;
        s_wt[tid] = wt;
      }
      __syncthreads();
      dn_compute(c, mfma, wm, stg, s_tok, s_wt, ytile);
      __syncthreads();
    }
#pragma unroll
    for (int s = 0; s < 8; ++s) wc[s] = wn[s];
    if (u + 1 == ue || (u + 1) / ne != r) {
      // this workgroup is done with group r: its tile goes to its slot
      const int first = run_of((unsigned long long)r * S), last = run_of((unsigned long long)r * S + P_last);
      const int slot = ri - first, nslots = last - first + 1;
      const int tile_f = kMaxBatch * kDnRows;
      float *slots = a.dn_part + (size_t)r * a.dn_slots * tile_f;
      const __amdgpu_buffer_rsrc_t rs = gu_rsrc(slots, a.dn_slots * tile_f);
      for (int q = tid; q < B * (kDnRows / 4); q += kBlock)
        __builtin_amdgcn_raw_buffer_store_b128(
            __builtin_bit_cast(v4u, *reinterpret_cast<const f32x4 *>(ytile + 4 * q)), rs,
            (slot * tile_f + 4 * q) * 4, 0, kGuSc1);
      wt_stores_complete();
      __syncthreads();
      if (tid == 0) {
        const unsigned prev = __hip_atomic_fetch_add(a.dn_cnt + r, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s_flag = prev == (unsigned)nslots - 1;
        if (s_flag) __hip_atomic_store(a.dn_cnt + r, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      __syncthreads();
      if (s_flag) {
        for (int q = tid; q < B * (kDnRows / 4); q += kBlock) {
          f32x4 y = {0.f, 0.f, 0.f, 0.f};
          for (int s0 = 0; s0 < nslots; s0 += 8) {
            f32x4 p[8];
#pragma unroll
            for (int j = 0; j < 8; ++j)
              p[j] = __builtin_bit_cast(
                  f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, (min(s0 + j, nslots - 1) * tile_f + 4 * q) * 4, 0,
                                                               kGuSc1));
#pragma unroll
            for (int j = 0; j < 8; ++j)
              if (s0 + j < nslots) y += p[j];
          }
          const int t = q / (kDnRows / 4), c4 = q % (kDnRows / 4);
          *reinterpret_cast<f32x4 *>(a.moe_out + (size_t)t * H + (size_t)r * kDnRows + 4 * c4) = y;
        }
      }
      for (int q = tid; q < kMaxBatch * kDnRows; q += kBlock) ytile[q] = 0.f;
      __syncthreads();
    }
  }
}

}  // namespace

hipError_t launch_batched(const BatchArgs &a, hipStream_t s, hipEvent_t (*ev)[2]) {
  const int n_wo = a.H / kProjRows;
  const int n_q = (a.Dq + kProjRows - 1) / kProjRows * a.qkv_split;
  const int n_rk = a.H / kBatchRtrK;
  hipError_t e;
  auto rec = [&](int i, int j) { return ev ? hipEventRecord(ev[i][j], s) : hipSuccess; };
#define DL_TRY(x) do { if ((e = (x)) != hipSuccess) return e; } while (0)
  DL_TRY(rec(0, 0));
  hipLaunchKernelGGL(proj_b, dim3(n_wo + n_q), dim3(kBlock), 0, s, a, n_wo);
  DL_TRY(hipGetLastError());
  DL_TRY(rec(0, 1));
  DL_TRY(rec(1, 0));
  hipLaunchKernelGGL(router_b, dim3((a.E + kBatchRtrExperts - 1) / kBatchRtrExperts, n_rk), dim3(kBlock), 0, s, a);
  DL_TRY(hipGetLastError());
  DL_TRY(rec(1, 1));
  DL_TRY(rec(2, 0));
  hipLaunchKernelGGL(topk_b, dim3(a.B), dim3(kBlock), 0, s, a, n_wo, n_rk);
  DL_TRY(hipGetLastError());
  DL_TRY(rec(2, 1));
  DL_TRY(rec(3, 0));
  hipLaunchKernelGGL(gateup_b, dim3(a.gu_grid), dim3(kBlock), 0, s, a);
  DL_TRY(hipGetLastError());
  DL_TRY(rec(3, 1));
  DL_TRY(rec(4, 0));
  hipLaunchKernelGGL(down_b, dim3(min(a.gu_grid, kDnMaxGrid)), dim3(kBlock), 0, s, a);
  DL_TRY(hipGetLastError());
  DL_TRY(rec(4, 1));
#undef DL_TRY
  return hipSuccess;
}

}  // namespace dl
