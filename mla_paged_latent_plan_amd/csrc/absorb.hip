// Weight absorption around the decode (vLLM mla_attention.py, forward_mqa and _v_up_proj; module
// docstring, "Data-Movement Friendly Approach"), as per-head bf16 GEMMs on MFMA:
//
//   mla_q_absorb: q[t, h, 0:L] = q_nope[t, h, :] . w_uk[h]^T, q[t, h, L:L+R] = q_pe[t, h, :]
//                 (w_uk [H, L, P]: the query's NoPE part moved into the latent space, and the
//                 decode's query assembled in place)
//   mla_v_up:     out[t, h, :] = o[t, h, :] . w_uv[h]^T (w_uv [H, V, L]: the decode's latent
//                 output moved back to the per-head value space)
//
// Both are C[t, n] = sum_k A[t, k] W[n, k] per head with k contiguous in A and W, so every MFMA
// operand is one 16-byte load per lane (no transposition). The kernels compute C^T tiles,
// D[n][t] = W[n, :] . A[t, :], on v_mfma_f32_16x16x32_bf16 with fp32 accumulation; each lane ends
// with four consecutive n of one t (bf16, round to nearest even): the tiled kernel stores them as
// 8 bytes, the weight-stationary kernel pairs lanes to store 16.
// DeepSeek-V3 shapes run the weight-stationary kernel below; other shapes the tiled one: a
// workgroup of four waves owns 64 n x 64 t of one head, wave w rows n0 + 16 w .. + 15 and all 64 t
// (four 16 x 16 accumulators), operands straight from global memory with the next k step's five
// loads issued before the current step's four MFMAs.
#include "layer_internal.h"

namespace mla {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kTileN = 64, kTileT = 64;

__device__ __forceinline__ uint32_t bf16_bits(float x) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)x);
}

__global__ __launch_bounds__(256) void absorb_gemm_kernel(GemmArgs a) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int h = blockIdx.z;
  const int n0 = blockIdx.y * kTileN + 16 * wave;
  const int t0 = blockIdx.x * kTileT;
  const int r16 = lane & 15, kq = 8 * (lane >> 4);  // operand row in the 16-row tile, k offset

  // W operand: row n0 + r16 of head h. A operands: rows t0 + 16 i + r16 (clamped to T - 1; the
  // clamped rows' results are not stored).
  const uint16_t* wp = a.w + ((int64_t)h * a.N + n0 + r16) * a.K + kq;
  const uint16_t* ap[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = min(t0 + 16 * i + r16, a.T - 1);
    ap[i] = a.a + (int64_t)t * a.a_t + (int64_t)h * a.a_h + kq;
  }
  f32x4 acc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

  bf16x8 wcur = *reinterpret_cast<const bf16x8*>(wp);
  bf16x8 acur[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) acur[i] = *reinterpret_cast<const bf16x8*>(ap[i]);
  for (int k = 32; k <= a.K; k += 32) {
    bf16x8 wnxt = wcur, anxt[4] = {acur[0], acur[1], acur[2], acur[3]};
    if (k < a.K) {
      wnxt = *reinterpret_cast<const bf16x8*>(wp + k);
#pragma unroll
      for (int i = 0; i < 4; ++i) anxt[i] = *reinterpret_cast<const bf16x8*>(ap[i] + k);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
      acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wcur, acur[i], acc[i], 0, 0, 0);
    wcur = wnxt;
#pragma unroll
    for (int i = 0; i < 4; ++i) acur[i] = anxt[i];
  }

  // acc[i][e] = D[n0 + 4 (lane >> 4) + e][t0 + 16 i + r16]
  const int n = n0 + 4 * (lane >> 4);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = t0 + 16 * i + r16;
    if (t < a.T) {
      const u32x2 v = {bf16_bits(acc[i][0]) | (bf16_bits(acc[i][1]) << 16),
                       bf16_bits(acc[i][2]) | (bf16_bits(acc[i][3]) << 16)};
      *reinterpret_cast<u32x2*>(a.c + (int64_t)t * a.c_t + (int64_t)h * a.c_h + n) = v;
    }
  }

  // the query's RoPE tail, copied after the latent columns by the first n-tile's workgroups
  if (a.pe != nullptr && blockIdx.y == 0) {
    const int chunks = a.R / 8;  // 16-byte pieces per row
    for (int idx = threadIdx.x; idx < kTileT * chunks; idx += blockDim.x) {
      const int t = t0 + idx / chunks, c = idx % chunks;
      if (t < a.T) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(a.pe + (int64_t)t * a.pe_t + (int64_t)h * a.pe_h + 8 * c);
        *reinterpret_cast<u32x4*>(a.c + (int64_t)t * a.c_t + (int64_t)h * a.c_h + a.N + 8 * c) = v;
      }
    }
  }
}

// Weight-stationary form: a workgroup (eight waves) holds NS rows of its head's weight matrix in
// LDS (NS x K bf16, rows padded by 16 bytes so that the 16 rows an MFMA operand reads sit in
// different banks) and streams a chunk of tokens past it: wave w takes 16-token tiles w, w + 8, ...
// of the chunk, reads their K-long rows once from global memory (the MFMA B operand; the next
// tile's rows are loaded while the current tile runs), and runs every k step against all NS / 16
// weight tiles read from LDS. Each weight byte then enters the
// compute unit once per token chunk and each token row once per weight slice, instead of once per
// 64 x 64 output tile. Used when the slice fits in LDS; NT accumulator tiles per wave.
template <int K, int NT>
__global__ __launch_bounds__(512) void absorb_ws_kernel(GemmArgs a, int t_chunk, int chunks,
                                                        int slices) {
  constexpr int kRow = 2 * K + 16;  // LDS bytes per weight row
  constexpr int NS = 16 * NT;       // weight rows (output columns) per workgroup
  __shared__ __attribute__((aligned(16))) uint8_t lds[NS * kRow];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  // Workgroups are dealt to the 8 XCDs round-robin: workgroup b runs on XCD b mod 8. All token
  // chunks of a (head, slice) share that XCD, so its L2 fetches the weight slice from memory once.
  const int x = blockIdx.x & 7, q = blockIdx.x >> 3;
  const int chunk = q % chunks, slice = (q / chunks) % slices;
  const int h = (q / chunks / slices) * 8 + x;
  if (h >= a.H) return;
  const int n0 = slice * NS;
  const int t_begin = chunk * t_chunk;
  const int t_end = min(a.T, t_begin + t_chunk);

  const int r16 = lane & 15, kq = 8 * (lane >> 4);
  // token rows of a tile (the MFMA B operand for every k step); rows past T repeat row T - 1
  auto load_tile = [&](int t0, bf16x8 (&av)[K / 32]) {
    const int t = min(t0 + r16, a.T - 1);
    const uint16_t* ap = a.a + (int64_t)t * a.a_t + (int64_t)h * a.a_h + kq;
#pragma unroll
    for (int ks = 0; ks < K / 32; ++ks) av[ks] = *reinterpret_cast<const bf16x8*>(ap + 32 * ks);
  };
  bf16x8 acur[K / 32], anxt[K / 32];
  int t0 = t_begin + 16 * wave;
  if (t0 < t_end) load_tile(t0, acur);  // in flight during the staging below

  // stage the weight slice (rows n0 .. n0 + NS - 1 of head h): each thread moves 16-byte pieces
  // c = tid + 512 j, eight loads in flight before their LDS stores
  {
    const uint8_t* src = reinterpret_cast<const uint8_t*>(a.w + ((int64_t)h * a.N + n0) * K);
    constexpr int kPieces = NS * (2 * K / 16);
    static_assert(kPieces % (512 * 8) == 0, "staging batches of eight pieces per thread");
#pragma unroll 1
    for (int j0 = 0; j0 < kPieces / 512; j0 += 8) {
      u32x4 v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int c = threadIdx.x + 512 * (j0 + j);
        v[j] = *reinterpret_cast<const u32x4*>(src + (int64_t)(c / (2 * K / 16)) * 2 * K + 16 * (c % (2 * K / 16)));
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int c = threadIdx.x + 512 * (j0 + j);
        *reinterpret_cast<u32x4*>(lds + (c / (2 * K / 16)) * kRow + 16 * (c % (2 * K / 16))) = v[j];
      }
    }
  }
  __syncthreads();

  for (; t0 < t_end; t0 += 16 * 8) {
    // the next tile's rows are in flight while this tile runs
    if (t0 + 16 * 8 < t_end) load_tile(t0 + 16 * 8, anxt);
    f32x4 acc[NT];
#pragma unroll
    for (int i = 0; i < NT; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < K / 32; ++ks) {
      const uint8_t* wrow = lds + r16 * kRow + 2 * (32 * ks + kq);
#pragma unroll
      for (int i = 0; i < NT; ++i) {
        const bf16x8 wv = *reinterpret_cast<const bf16x8*>(wrow + 16 * i * kRow);
        acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wv, acur[ks], acc[i], 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);  // keep the next step's LDS reads after these MFMAs
    }
    // acc[i][e] = D[n0 + 16 i + 4 g + e][t0 + r16], g = lane >> 4. Lanes g and g ^ 1 swap halves
    // of a pair of tiles (i, i + 1) so that each holds eight consecutive columns: even g
    // 16 i + 4 g .. + 7, odd g 16 (i + 1) + 4 (g - 1) .. + 7, one 16-byte store each.
    {
      const int g = lane >> 4;
      const bool odd = g & 1;
      uint16_t* cp = a.c + (int64_t)(t0 + r16) * a.c_t + (int64_t)h * a.c_h + n0;
#pragma unroll
      for (int i = 0; i < NT; i += 2) {
        const u32x2 v0 = {bf16_bits(acc[i][0]) | (bf16_bits(acc[i][1]) << 16),
                          bf16_bits(acc[i][2]) | (bf16_bits(acc[i][3]) << 16)};
        const u32x2 v1 = {bf16_bits(acc[i + 1][0]) | (bf16_bits(acc[i + 1][1]) << 16),
                          bf16_bits(acc[i + 1][2]) | (bf16_bits(acc[i + 1][3]) << 16)};
        const u32x2 send = odd ? v0 : v1;
        const u32x2 recv = {(uint32_t)__shfl_xor((int)send[0], 16, 64),
                            (uint32_t)__shfl_xor((int)send[1], 16, 64)};
        const u32x4 w = odd ? u32x4{recv[0], recv[1], v1[0], v1[1]}
                            : u32x4{v0[0], v0[1], recv[0], recv[1]};
        const int col = odd ? 16 * (i + 1) + 4 * (g - 1) : 16 * i + 4 * g;
        if (t0 + r16 < a.T) *reinterpret_cast<u32x4*>(cp + col) = w;
      }
    }
#pragma unroll
    for (int ks = 0; ks < K / 32; ++ks) acur[ks] = anxt[ks];
  }

  // the query's RoPE tail, copied after the latent columns by the first slice's workgroups
  if (a.pe != nullptr && slice == 0) {
    const int pieces = a.R / 8;
    for (int idx = threadIdx.x; idx < (t_end - t_begin) * pieces; idx += blockDim.x) {
      const int tt = t_begin + idx / pieces, c = idx % pieces;
      const u32x4 v = *reinterpret_cast<const u32x4*>(a.pe + (int64_t)tt * a.pe_t + (int64_t)h * a.pe_h + 8 * c);
      *reinterpret_cast<u32x4*>(a.c + (int64_t)tt * a.c_t + (int64_t)h * a.c_h + a.N + 8 * c) = v;
    }
  }
}

// Weight-stationary launch for (K, slice rows): token chunks as long as possible (each chunk
// re-reads the weight slice) while the grid still fills every compute unit; chunks are whole
// 16-token tiles.
template <int K, int NT>
hipError_t launch_ws(const GemmArgs& a, hipStream_t s) {
  constexpr int NS = 16 * NT;
  static_assert(NT % 2 == 0, "output columns are stored in pairs of 16-column tiles");
  // workgroups one compute unit can hold (LDS): two for the 70 KB query-absorption slice
  constexpr int kPerCu = (NS * (2 * K + 16) <= 80 * 1024) ? 2 : 1;
  const int slices = a.N / NS;
  int t_chunk = (a.T + 15) / 16 * 16;
  while (t_chunk > 16 && (int64_t)((a.T + t_chunk - 1) / t_chunk) * slices * a.H < 256 * kPerCu)
    t_chunk = (t_chunk / 2 + 15) / 16 * 16;
  const int chunks = (a.T + t_chunk - 1) / t_chunk;
  const int64_t grid = (int64_t)chunks * slices * ((a.H + 7) / 8) * 8;
  hipLaunchKernelGGL((absorb_ws_kernel<K, NT>), dim3((unsigned)grid), dim3(512), 0, s, a, t_chunk,
                     chunks, slices);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_absorb_gemm(const GemmArgs& a, hipStream_t s) {
  if (a.T <= 0) return hipSuccess;
  // DeepSeek-V3 shapes run weight-stationary: query absorption (K = 128, 512 columns in slices of
  // 256) and value up-projection (K = 512, all 128 columns)
  if (a.K == 128 && a.N % 256 == 0) return launch_ws<128, 16>(a, s);
  if (a.K == 512 && a.N % 128 == 0) return launch_ws<512, 8>(a, s);
  const dim3 grid((unsigned)((a.T + kTileT - 1) / kTileT), (unsigned)(a.N / kTileN), (unsigned)a.H);
  hipLaunchKernelGGL(absorb_gemm_kernel, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace mla
