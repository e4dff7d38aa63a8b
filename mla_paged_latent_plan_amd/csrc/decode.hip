// mla_decode kernel for gfx950: absorbed-form MLA decode over a paged latent cache.
//
// What it computes (vLLM mla_attention.py module docstring, "Data-Movement Friendly Approach"):
// all heads of a query group attend over the same latent rows, K = [kv_c, k_pe] (d_qk wide) and
// V = kv_c (the first 512 columns). Per split (a run of 64-row blocks of one group, from the
// plan) a workgroup produces either the final bf16 O and natural-log LSE, or a partial
// (bf16 O normalised by its own denominator, fp32 LSE without the sink) for mla_combine. On
// request the 64-row kernel also writes each row's largest scaled score (the max_logits output of
// the FlashMLA wrapper's flash_mla_sparse_fwd), final or per split.
//
// Mapping onto CDNA4:
// - Workgroup = 4 waves; the group's query rows (heads, times tokens when q_len > 1) are the
//   N dimension of S^T = K Q^T and of O^T = V^T P^T, so one LDS copy of a KV block serves every
//   head of the tile. A wave owns HW query rows (Q^T kept in VGPRs) and KVW rows of each block;
//   waves that split a block's rows (WN > 1) keep separate softmax states merged at the end.
// - KV rows are gathered page by page with global_load_lds_dwordx4 (no VGPR staging), one row
//   (1 KB) or eight RoPE tails per instruction, into a double-buffered LDS stage of 64 rows.
//   The latent part uses a padded row stride (1040 B); S^T tile row m maps to LDS row rho(m) so
//   that both the QK^T operand reads (ds_read_b128) and the transposed V reads
//   (ds_read_b64_tr_b16) hit distinct banks with affine addresses. RoPE tails are XOR-swizzled.
// - QK^T and PV are v_mfma_f32_16x16x32_bf16 (16x16x16 when a wave owns only 16 rows of a
//   block). The S^T accumulator layout is directly the B operand of PV, so P never leaves
//   registers; V^T comes from the transposed LDS read.
// - Online softmax in base 2 with a lazily moved reference maximum: O is rescaled only when a
//   row's maximum grows by more than 2^16, which keeps the 256 accumulator registers untouched in
//   the common case. Row statistics are per lane (the head index runs along lanes).
// - Masked rows (past the group's rows, invalid indices, pages outside the cache) are gathered
//   from the plan's zero row, so no NaN from unused cache bytes can reach the accumulators.
#include <type_traits>

#include "mla_internal.h"

namespace mla {

namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

// Output and partial stores of the 64- and 128-row kernels as inline assembly, with device scope
// (sc1): each write goes through the XCD's L2 to the device's coherence point as it is made, so
// the release at the kernel's end has few dirty L2 lines left to write back before the next
// kernel may start (about 2 us off a 110 us step; the 16-row kernel's stores are faster without
// it). The compiler's wait-count pass does not see these stores, so it does not make later
// register writes wait for them (with LDS-DMA transfers in flight, such a wait would also hold
// for every transfer); nothing in a decode kernel reads what it stores. One wait state after each
// guards the store-data hazard.
__device__ __forceinline__ void st_global_b128(void* p, const u32x4& v) {
  asm volatile("global_store_dwordx4 %0, %1, off sc1\n\ts_nop 1" :: "v"(p), "v"(v) : "memory");
}
__device__ __forceinline__ void st_global_b32(void* p, float v) {
  asm volatile("global_store_dword %0, %1, off sc1\n\ts_nop 1" :: "v"(p), "v"(v) : "memory");
}
#define LDS_AS __attribute__((address_space(3)))

constexpr int kThreads = 256;
constexpr int kRowStrideA = 1056;            // latent part: 1 KB + 32 B padding (bank spread)
constexpr int kStageA = kBlockRows * kRowStrideA;
constexpr int kStageB = kBlockRows * 128;    // RoPE tails (64 bf16), XOR-swizzled
constexpr float kNegInf = -__builtin_inff();
// Lazy rescale threshold (log2 units): the reference maximum of a row moves, and O is rescaled, only
// when the row maximum exceeds it by more than 2^64. Probabilities then stay below 2^64 (bf16 keeps
// its relative rounding at any magnitude) and O and l below 2^64 x rows x max|V|: inside fp32 for
// max|V| up to 2^(64 - log2 rows) (2^47 at 128K rows). A smaller threshold rescales far more often
// on fp8 rows with ue8m0 scales, whose scores spread over tens of log2 units (each rescale touches
// all of a wave's O accumulators).
constexpr float kTau = 64.0f;
// The 16-row kernel reads each KV row once and takes it with the streaming (non-temporal) cache
// policy (≈ 4 % faster at 16 heads). The 64-row kernel keeps the default policy: the second row
// tile of a unit reads the same rows and finds them in L2 (the policy measured neutral there).
constexpr bool kRowsNT = true;

constexpr int kMergeStride = kDv + 4;  // floats per O row in the 16-row kernel's merge scratch

template <int HW_, int WN_, int DQK_>
struct Cfg {
  static constexpr int HW = HW_;             // query rows per wave
  static constexpr int WN = WN_;             // waves sharing a head tile (splitting block rows)
  static constexpr int WM = 4 / WN;          // head tiles per workgroup
  static constexpr int DQK = DQK_;
  static constexpr int M_TILE = HW * WM;
  static constexpr int NT = HW / 16;
  static constexpr int KVW = kBlockRows / WN;
  static constexpr int SUB = KVW >= 32 ? 32 : 16;  // rows per softmax/PV step
  static constexpr int NSUB = KVW / SUB;
  static constexpr int KT = SUB / 16;              // 16-row S^T tiles per step
  static constexpr int KS = DQK / 32;
  static constexpr bool HAS_B = DQK > 512;
  static constexpr int STAGE = kStageA + (HAS_B ? kStageB : 0);
  static constexpr int RI_OFF = 2 * STAGE;  // row entries: block-table [4][64], index [8][64]
  static constexpr int LDS = RI_OFF + 12 * 256;
  static constexpr int NB = 16 + (HAS_B ? 2 : 0) + 1;  // memory instructions per dense bundle
  static_assert(WN == 1 || 4 * HW * kMergeStride * 4 + 8 * HW * 4 + M_TILE * WN * 4 <= RI_OFF,
                "merge scratch must fit in the stage buffers");
};

// S^T tile row m (MFMA lane index) -> LDS row within the 16-row tile. With the 1056-byte row
// stride the identity order keeps both the K-operand reads and the transposed V reads free of
// bank conflicts.
__device__ __forceinline__ int rho(int m) { return m; }
__device__ __forceinline__ int swz_b(int row) { return (row >> 1) & 7; }

typedef LDS_AS uint8_t* lds_ptr;

__device__ __forceinline__ bf16x8 lds_read_b128(lds_ptr base, uint32_t off) {
  return *reinterpret_cast<const LDS_AS bf16x8*>(base + off);
}
// The restrict-qualified inlined helper gives the transposed read alias metadata. Without it the
// compiler's wait-count pass cannot tell the read from in-flight LDS-DMA writes and drains every
// outstanding global load before it; the kernels order DMA and reads with explicit waits instead.
__device__ __forceinline__ bf16x4 lds_read_tr_nz(LDS_AS bf16x4* __restrict__ p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16(p);
}
__device__ __forceinline__ bf16x4 lds_read_tr(lds_ptr base, uint32_t off) {
  return lds_read_tr_nz(reinterpret_cast<LDS_AS bf16x4*>(base + off));
}

__device__ __forceinline__ float wave_max_groups(float v) {
  v = fmaxf(v, __shfl_xor(v, 16, 64));
  v = fmaxf(v, __shfl_xor(v, 32, 64));
  return v;
}
__device__ __forceinline__ float wave_sum_groups(float v) {
  v += __shfl_xor(v, 16, 64);
  v += __shfl_xor(v, 32, 64);
  return v;
}

// Same reductions across the four 16-lane rows with the VALU lane swaps (no LDS round trip).
__device__ __forceinline__ float rows_max(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float rows_sum(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// ue8m0 scale byte -> 2^(s - 127) as a float (byte 0 is the subnormal 2^-127, byte 255 is NaN).
__device__ __forceinline__ float ue8m0_f32(uint32_t s) {
  const uint32_t bits = (s == 0u) ? 0x00400000u : ((s == 255u) ? 0x7FC00000u : (s << 23));
  return __uint_as_float(bits);
}
// Eight e4m3 bytes (little-endian order in w) of one scale group -> bf16, times the group scale.
// The product of an e4m3 value and a power of two is exact in bf16.
__device__ __forceinline__ bf16x8 fp8x8_scaled(uint32_t w0, uint32_t w1, float sc) {
  const auto a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, sc, false);
  const auto b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, sc, true);
  const auto c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, sc, false);
  const auto d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, sc, true);
  return bf16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}
// fp8 latent region: 512-byte rows, 16-byte chunk c of row r stored at chunk c ^ swz_n(r). Keeps
// the K-operand reads (16 consecutive rows) free of bank conflicts.
__device__ __forceinline__ int swz_n(int row) { return (row & 15) ^ ((row >> 4) << 3); }

__device__ __forceinline__ uint64_t readlane64(uint64_t v, int lane) {
  uint32_t lo = __builtin_amdgcn_readlane((uint32_t)v, lane);
  uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(v >> 32), lane);
  return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ uint16_t f2bf(float x) {
  __bf16 b = (__bf16)x;
  return __builtin_bit_cast(uint16_t, b);
}

// LDS-DMA as inline assembly (M0 = wave-uniform LDS base, one 16- or 4-byte element per lane).
// Seeing the DMA builtin in a loop, the compiler's wait-count pass falls back to waiting for every
// outstanding LDS read before each use; the kernels that use these helpers order their DMA and LDS
// reads with explicit vmcnt waits and barriers instead. M0 has no other user in those kernels.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// NT = streaming (non-temporal) cache policy: with it one CU streams ≈ 28 GB/s from HBM while the
// whole chip streams, against ≈ 23 GB/s with the default policy.
template <bool NT = false>
__device__ __forceinline__ void dma_x4(const void* src, uint32_t lds_addr) {
  if constexpr (NT)
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt"
                 :: "v"(src), "s"(lds_addr) : "memory", "m0");
  else
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                 :: "v"(src), "s"(lds_addr) : "memory", "m0");
}
// row (wave-uniform, scalar registers) + lane_off
template <bool NT = false>
__device__ __forceinline__ void dma_x4s(uint32_t lane_off, uint64_t row, uint32_t lds_addr) {
  if constexpr (NT)
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 nt"
                 :: "v"(lane_off), "s"(row), "s"(lds_addr) : "memory", "m0");
  else
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                 :: "v"(lane_off), "s"(row), "s"(lds_addr) : "memory", "m0");
}
template <bool NT = false>
__device__ __forceinline__ void dma_x1(const void* src, uint32_t lds_addr) {
  if constexpr (NT)
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off nt"
                 :: "v"(src), "s"(lds_addr) : "memory", "m0");
  else
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"
                 :: "v"(src), "s"(lds_addr) : "memory", "m0");
}
#pragma clang diagnostic pop
__device__ __forceinline__ uint32_t lds_addr(lds_ptr p) { return (uint32_t)(uintptr_t)p; }

// Workgroup barrier for LDS hand-offs only: unlike __syncthreads() it does not wait for
// outstanding global loads, so the next block's LDS-DMA stays in flight across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

template <class C>
struct Decoder {
  const DecodeArgs& a;
  lds_ptr sm;
  int lane, wave, wm, wn;
  // current split
  int g, b, L, j0, n, kb, ke;

  __device__ Decoder(const DecodeArgs& args, lds_ptr base) : a(args), sm(base) {
    lane = threadIdx.x & 63;
    wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform: scalar registers
    wm = wave / C::WN;
    wn = wave % C::WN;
  }

  __device__ __forceinline__ uint32_t stage_a(int st) const { return st * C::STAGE; }
  __device__ __forceinline__ uint32_t stage_b(int st) const { return st * C::STAGE + kStageA; }

  // Row entries of block x travel by LDS-DMA into workgroup rings (block-table entries of four
  // blocks, index entries of eight), so no register ever waits on an in-flight load. Wave w fetches
  // the entries of rows [16w, 16w + 16); addresses are clamped and the values validated when used.
  __device__ __forceinline__ uint32_t pg_slot(int x) const { return C::RI_OFF + (x & 3) * 256; }
  __device__ __forceinline__ uint32_t ix_slot(int x) const { return C::RI_OFF + 1024 + (x & 7) * 256; }
  __device__ __forceinline__ void dma_entry(const int32_t* src, uint32_t slot) const {
    if (lane < 16) dma_x1(src, lds_addr(sm + slot + 64 * wave));
  }
  __device__ __forceinline__ int ri_read(uint32_t slot, int row) const {
    return *reinterpret_cast<const LDS_AS int*>(sm + slot + 4 * row);
  }
  __device__ __forceinline__ int erow() const { return (16 * wave + lane) & 63; }
  __device__ __forceinline__ void idx_fetch(int x) const {
    const int k = min(x * kBlockRows + erow(), a.topk - 1);
    dma_entry(a.indices + (int64_t)g * a.topk + max(k, 0), ix_slot(x));
  }
  // logical position (dense) or index value (sparse) of row `row` of block x
  __device__ __forceinline__ int row_j(int x, int row) const {
    return (a.topk > 0) ? ri_read(ix_slot(x), row) : j0 + x * kBlockRows + row;
  }
  __device__ __forceinline__ void page_fetch(int x) const {
    const int pi = min(max(row_j(x, erow()) >> a.ps_log2, 0), a.max_pages - 1);
    dma_entry(a.block_table + (int64_t)b * a.max_pages + pi, pg_slot(x));
  }
  // Global address of row `lane` of block x; invalid rows read the zero row.
  __device__ __forceinline__ uint64_t row_base(int x, int* valid) const {
    const int j = row_j(x, lane);
    const int page = ri_read(pg_slot(x), lane);
    const int k = x * kBlockRows + lane;
    bool ok = k < n && (j >> a.ps_log2) < a.max_pages;
    if (a.topk > 0) ok = ok && j >= 0 && j < L;
    ok = ok && page >= 0 && (int64_t)page < a.num_pages;
    *valid = ok;
    if (!ok) return (uint64_t)(uintptr_t)a.zero_row;
    const int slot = j & ((1 << a.ps_log2) - 1);
    return (uint64_t)(uintptr_t)(a.cache + (int64_t)page * a.page_stride + (int64_t)slot * a.row_bytes);
  }

  // Bundle x: the LDS-DMA of block x into stage x & 1 (wave w moves rows [16w, 16w + 16)), the
  // block-table entries of block x + 2 and, with index lists, the index entries of block x + 4.
  // Every wave issues the same C::NB (+1 sparse) memory instructions, so "bundle x has landed" is an
  // exact vmcnt. Returns the valid-row mask of block x.
  __device__ __forceinline__ uint64_t bundle(int x) const {
    int v;
    const uint64_t base = row_base(x, &v);
    const uint64_t vm = __ballot(v);
    const uint32_t sa = stage_a(x & 1);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int r = wave * 16 + i;
      dma_x4s<kRowsNT>(16 * lane, readlane64(base, r), lds_addr(sm + sa + r * kRowStrideA));
    }
    if constexpr (C::HAS_B) {
      const uint32_t sb = stage_b(x & 1);
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const int k = wave * 2 + kk;
        const int r = 8 * k + (lane >> 3);
        const int c = (lane & 7) ^ swz_b(r);
        const uint32_t lo = __shfl((uint32_t)base, r, 64);
        const uint32_t hi = __shfl((uint32_t)(base >> 32), r, 64);
        const uint8_t* src = reinterpret_cast<const uint8_t*>((uintptr_t)(((uint64_t)hi << 32) | lo)) +
                             1024 + 16 * c;
        dma_x4<kRowsNT>(src, lds_addr(sm + sb + k * 1024));
      }
    }
    page_fetch(x + 2);
    if (a.topk > 0) idx_fetch(x + 4);
    return vm;
  }

  __device__ void run_split(int s, int mt) {
    const int32_t* plan = a.plan;
    const int32_t* rec = plan + a.splits_off + 4 * (int64_t)s;
    g = rec[0];
    kb = rec[1];
    ke = rec[2];
    j0 = plan[a.grp_rows_off + 2 * g];
    n = plan[a.grp_rows_off + 2 * g + 1];
    const int nsplit = plan[a.grp_ptr_off + g + 1] - plan[a.grp_ptr_off + g];
    b = (a.topk > 0) ? g / a.Sq : g;
    L = a.seqlens[b];

    const int row0 = mt * C::M_TILE + wm * C::HW;  // first query row of this wave
    const int nl = lane & 15, gl = lane >> 4;

    // ---- Q^T operand registers ------------------------------------------------------------
    bf16x8 qr[C::NT][C::KS];
#pragma unroll
    for (int nt = 0; nt < C::NT; ++nt) {
      const int r = row0 + nt * 16 + nl;
      const bool ok = r < a.R;
      const bf16x8* src = reinterpret_cast<const bf16x8*>(
          a.q + ((int64_t)g * a.R + (ok ? r : 0)) * C::DQK + 8 * gl);
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
        bf16x8 v = src[4 * ks];
        if (!ok) v = bf16x8{};
        qr[nt][ks] = v;
      }
    }
    // query position of each lane's rows (dense masks)
    int qpos[C::NT];
#pragma unroll
    for (int nt = 0; nt < C::NT; ++nt) {
      const int r = row0 + nt * 16 + nl;
      const int t = (a.topk > 0) ? 0 : (r / a.H);
      qpos[nt] = L - a.Sq + t;
    }

    float m_ref[C::NT], l_acc[C::NT];
    f32x4 o[C::NT][kDv / 16];
#pragma unroll
    for (int nt = 0; nt < C::NT; ++nt) {
      m_ref[nt] = kNegInf;
      l_acc[nt] = 0.f;
#pragma unroll
      for (int dt = 0; dt < kDv / 16; ++dt) o[nt][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    // ---- prologue: index entries of blocks kb..kb+3, block-table entries of kb, kb+1 (in flight
    // together with the Q loads), then bundle kb
    const bool sparse = a.topk > 0;
    if (sparse) {
#pragma unroll
      for (int i = 0; i < 4; ++i) idx_fetch(kb + i);
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      lds_barrier();
    }
    page_fetch(kb);
    page_fetch(kb + 1);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    lds_barrier();
    // The Q registers are complete here. Naming them in an asm statement makes the compiler place
    // its own wait for the Q loads now, before any row transfer is in flight: its wait counts do
    // not see the inline-assembly transfers, so a wait placed later would also wait for those.
#pragma unroll
    for (int nt = 0; nt < C::NT; ++nt)
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) asm volatile("" : "+v"(qr[nt][ks]));
    uint64_t vmask_next = bundle(kb);

    const bool dense_mask = (a.topk == 0) && (a.causal || a.window > 0);
    for (int blk = kb; blk < ke; ++blk) {
      const int cur = blk & 1;
      const uint64_t vmask = vmask_next;
      // bundle blk + 1 goes into the stage of block blk - 1, released at the last barrier; then
      // wait for this wave's bundle blk, and the barrier makes every wave's transfers visible
      if (blk + 1 < ke) {
        vmask_next = bundle(blk + 1);
        if (sparse) asm volatile("s_waitcnt vmcnt(%0)" :: "n"(C::NB + 1) : "memory");
        else asm volatile("s_waitcnt vmcnt(%0)" :: "n"(C::NB) : "memory");
      } else {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      }
      lds_barrier();

      const uint32_t sa = stage_a(cur);
      const uint32_t sb = stage_b(cur);
#pragma unroll
      for (int sub = 0; sub < C::NSUB; ++sub) {
        const int rbase = wn * C::KVW + sub * C::SUB;  // first stage row of this step

        // ---- S^T = K Q^T -------------------------------------------------------------------
        f32x4 sacc[C::KT][C::NT];
#pragma unroll
        for (int kt = 0; kt < C::KT; ++kt)
#pragma unroll
          for (int nt = 0; nt < C::NT; ++nt) sacc[kt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
        uint32_t kaddr[C::KT];
#pragma unroll
        for (int kt = 0; kt < C::KT; ++kt)
          kaddr[kt] = sa + (rbase + 16 * kt + rho(nl)) * kRowStrideA + 16 * gl;
        // K operand of step ks for tile kt: latent part (affine) or RoPE tail (swizzled)
        auto k_operand = [&](int kt, int ks) -> bf16x8 {
          if (ks < 16) return lds_read_b128(sm, kaddr[kt] + 64 * ks);
          const int row = rbase + 16 * kt + rho(nl);
          const int c = (4 * (ks - 16) + gl) ^ swz_b(row);
          return lds_read_b128(sm, sb + row * 128 + 16 * c);
        };
        // D - 1 steps of operands in flight ahead of the MFMAs that consume the oldest
        constexpr int D = 4;
        bf16x8 ka[D][C::KT];
#pragma unroll
        for (int i = 0; i < D - 1; ++i)
#pragma unroll
          for (int kt = 0; kt < C::KT; ++kt) ka[i][kt] = k_operand(kt, i);
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) {
          if (ks + D - 1 < C::KS) {
#pragma unroll
            for (int kt = 0; kt < C::KT; ++kt) ka[(ks + D - 1) % D][kt] = k_operand(kt, ks + D - 1);
          }
#pragma unroll
          for (int kt = 0; kt < C::KT; ++kt)
#pragma unroll
            for (int nt = 0; nt < C::NT; ++nt)
              sacc[kt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[ks % D][kt], qr[nt][ks],
                                                                     sacc[kt][nt], 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
        }

        // ---- masks -------------------------------------------------------------------------
        const bool tail = blk * kBlockRows + rbase + C::SUB > n;
        bool need_mask = tail || dense_mask;
        if (a.topk > 0) need_mask = (vmask != ~0ull);
        if (need_mask) {
#pragma unroll
          for (int kt = 0; kt < C::KT; ++kt)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int row = rbase + 16 * kt + rho(4 * gl + e);
              const int k = blk * kBlockRows + row;
#pragma unroll
              for (int nt = 0; nt < C::NT; ++nt) {
                bool ok;
                if (a.topk > 0) {
                  ok = (vmask >> row) & 1;
                } else {
                  const int j = j0 + k;
                  ok = k < n;
                  if (a.causal) ok = ok && j <= qpos[nt];
                  if (a.window > 0) ok = ok && j >= qpos[nt] - a.window + 1;
                }
                if (!ok) sacc[kt][nt][e] = kNegInf;
              }
            }
        }

        // ---- online softmax (base 2, lazy reference max) ------------------------------------
        bool need_rescale = false;
        float m_new[C::NT];
#pragma unroll
        for (int nt = 0; nt < C::NT; ++nt) {
          float mx = kNegInf;
#pragma unroll
          for (int kt = 0; kt < C::KT; ++kt)
#pragma unroll
            for (int e = 0; e < 4; ++e) mx = fmaxf(mx, sacc[kt][nt][e]);
          mx = wave_max_groups(mx);
          m_new[nt] = mx * a.scale_log2;  // -inf stays -inf (scale > 0)
          need_rescale |= (m_new[nt] > m_ref[nt] + kTau);
        }
        if (__any(need_rescale)) {
#pragma unroll
          for (int nt = 0; nt < C::NT; ++nt) {
            const bool up = m_new[nt] > m_ref[nt] + kTau;
            const float alpha = up ? exp2f(m_ref[nt] - m_new[nt]) : 1.f;  // m_ref=-inf -> 0
            if (up) m_ref[nt] = m_new[nt];
            l_acc[nt] *= alpha;
#pragma unroll
            for (int dt = 0; dt < kDv / 16; ++dt) {
              o[nt][dt] *= alpha;
              __builtin_amdgcn_sched_barrier(0);  // one tile out of the accumulators at a time
            }
          }
        }
        // P = exp2(s * scale_log2 - m_ref), packed as the B operand of PV
        bf16x8 p8[C::NT];
        bf16x4 p4[C::NT];
#pragma unroll
        for (int nt = 0; nt < C::NT; ++nt) {
          const float mu = (m_ref[nt] == kNegInf) ? 0.f : m_ref[nt];
          float lsum = 0.f;
#pragma unroll
          for (int kt = 0; kt < C::KT; ++kt) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float pv = exp2f(__builtin_fmaf(sacc[kt][nt][e], a.scale_log2, -mu));
              lsum += pv;
              const __bf16 pb = (__bf16)pv;
              if constexpr (C::SUB == 32) p8[nt][kt * 4 + e] = pb;
              else p4[nt][e] = pb;
            }
          }
          l_acc[nt] += lsum;
        }

        // ---- O^T += V^T P^T ----------------------------------------------------------------
        // lane (i, g): transposed-read row rho(4g + i/4) of the tile, columns 16 dt + 4 (i % 4)
        const uint32_t vbase = sa + (rbase + rho(4 * gl + ((lane & 15) >> 2))) * kRowStrideA +
                               8 * (lane & 3);
        if constexpr (C::SUB == 32) {
          auto v_operand = [&](int dt) -> bf16x8 {
            const uint32_t ad = vbase + 32 * dt;
            const bf16x4 v0 = lds_read_tr(sm, ad);
            const bf16x4 v1 = lds_read_tr(sm, ad + 16 * kRowStrideA);
            return __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
          };
          bf16x8 va[D];
#pragma unroll
          for (int i = 0; i < D - 1; ++i) va[i] = v_operand(i);
#pragma unroll
          for (int dt = 0; dt < kDv / 16; ++dt) {
            if (dt + D - 1 < kDv / 16) va[(dt + D - 1) % D] = v_operand(dt + D - 1);
#pragma unroll
            for (int nt = 0; nt < C::NT; ++nt)
              o[nt][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[dt % D], p8[nt], o[nt][dt],
                                                                  0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
          }
        } else {
          bf16x4 va[D];
#pragma unroll
          for (int i = 0; i < D - 1; ++i) va[i] = lds_read_tr(sm, vbase + 32 * i);
#pragma unroll
          for (int dt = 0; dt < kDv / 16; ++dt) {
            if (dt + D - 1 < kDv / 16) va[(dt + D - 1) % D] = lds_read_tr(sm, vbase + 32 * (dt + D - 1));
#pragma unroll
            for (int nt = 0; nt < C::NT; ++nt)
              o[nt][dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va[dt % D], p4[nt], o[nt][dt],
                                                                    0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      }
      lds_barrier();  // every wave done with stage cur (bundle blk + 2 goes there)
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // nothing in flight (also for empty splits)
    lds_barrier();  // all waves done with the stage buffers (reused by the merge below)

    // ---- epilogue ----------------------------------------------------------------------------
    const bool final_out = (nsplit == 1);
    if constexpr (C::WN == 1) {
#pragma unroll
      for (int nt = 0; nt < C::NT; ++nt) {
        const float lt = wave_sum_groups(l_acc[nt]);
        const int r = row0 + nt * 16 + nl;
        write_row(s, r, m_ref[nt], lt, o[nt], final_out);
      }
    } else {
      // merge the WN partial states of each head tile through LDS; O rows are padded by 16 bytes
      // so that the 16 rows a wave writes with one instruction fall in different banks. The
      // barriers order LDS only: the output stores stay in flight across them.
      constexpr int kSo = kMergeStride;
      LDS_AS float* so = reinterpret_cast<LDS_AS float*>(sm);  // [wave][HW][kSo] O
      LDS_AS float* sml = so + 4 * C::HW * kSo;                 // [wave][HW] m, then l
#pragma unroll
      for (int nt = 0; nt < C::NT; ++nt) {
        const float lt = wave_sum_groups(l_acc[nt]);
        const int hrow = nt * 16 + nl;
        if (gl == 0) {
          sml[wave * C::HW + hrow] = m_ref[nt];
          sml[4 * C::HW + wave * C::HW + hrow] = lt;
        }
#pragma unroll
        for (int dt = 0; dt < kDv / 16; ++dt) {
          LDS_AS f32x4* dst =
              reinterpret_cast<LDS_AS f32x4*>(so + (wave * C::HW + hrow) * kSo + dt * 16 + 4 * gl);
          *dst = o[nt][dt];
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      lds_barrier();
      // per-row merge weights (the output normalisation folded in) and the row's LSE
      LDS_AS float* wts = sml + 8 * C::HW;  // [M_TILE][WN]
      if (threadIdx.x < C::M_TILE) {
        const int row = threadIdx.x;
        const int tm = row / C::HW, hrow = row % C::HW;
        float ms[C::WN], cw[C::WN];
        float mstar = kNegInf;
#pragma unroll
        for (int w = 0; w < C::WN; ++w) {
          ms[w] = sml[(tm * C::WN + w) * C::HW + hrow];
          mstar = fmaxf(mstar, ms[w]);
        }
        float lstar = 0.f;
#pragma unroll
        for (int w = 0; w < C::WN; ++w) {
          cw[w] = (ms[w] == kNegInf) ? 0.f : exp2f(ms[w] - mstar);
          lstar += cw[w] * sml[4 * C::HW + (tm * C::WN + w) * C::HW + hrow];
        }
        const int r = mt * C::M_TILE + row;
        float scale = 0.f;
        if (r < a.R) {
          float lse_nat;
          row_norm(r, mstar, lstar, final_out, &lse_nat, &scale);
          if (final_out) a.lse[lse_index(r)] = lse_nat;
          else a.part_lse[(int64_t)s * a.R + r] = lse_nat;
        }
#pragma unroll
        for (int w = 0; w < C::WN; ++w) wts[row * C::WN + w] = cw[w] * scale;
      }
      lds_barrier();
      // each thread: float4 column threadIdx.x % 128 of rows threadIdx.x / 128 + 2i; every LDS read
      // is issued before the first store
      constexpr int NI = C::M_TILE * (kDv / 4) / kThreads;
      const int c4 = threadIdx.x % (kDv / 4);
      f32x4 acc[NI];
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int row = (threadIdx.x + i * kThreads) / (kDv / 4);
        const int tm = row / C::HW, hrow = row % C::HW;
        acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int w = 0; w < C::WN; ++w) {
          const int wv = tm * C::WN + w;
          const f32x4 v = *reinterpret_cast<LDS_AS f32x4*>(so + (wv * C::HW + hrow) * kSo + 4 * c4);
          acc[i] += wts[row * C::WN + w] * v;
        }
      }
      uint16_t* dst0 = final_out ? a.out + (int64_t)g * a.R * kDv : a.part_o + (int64_t)s * a.R * kDv;
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int r = mt * C::M_TILE + (threadIdx.x + i * kThreads) / (kDv / 4);
        if (r < a.R) {
          uint2 w2;
          w2.x = (uint32_t)f2bf(acc[i][0]) | ((uint32_t)f2bf(acc[i][1]) << 16);
          w2.y = (uint32_t)f2bf(acc[i][2]) | ((uint32_t)f2bf(acc[i][3]) << 16);
          *reinterpret_cast<uint2*>(dst0 + (int64_t)r * kDv + 4 * c4) = w2;
        }
      }
      lds_barrier();  // scratch reused by the next split
    }
  }

  // Final or partial output of one query row from a lane's O^T registers (WN == 1 path).
  __device__ __forceinline__ void write_row(int s, int r, float m2, float l, const f32x4* orow,
                                            bool final_out) const {
    if (r >= a.R) return;
    const int gl = lane >> 4;
    float lse_nat, scale;
    row_norm(r, m2, l, final_out, &lse_nat, &scale);
    if (final_out) {
      uint16_t* dst = a.out + ((int64_t)g * a.R + r) * kDv + 4 * gl;
#pragma unroll
      for (int dt = 0; dt < kDv / 16; ++dt) {
        const f32x4 v = orow[dt] * scale;
        uint2 w;
        w.x = (uint32_t)f2bf(v[0]) | ((uint32_t)f2bf(v[1]) << 16);
        w.y = (uint32_t)f2bf(v[2]) | ((uint32_t)f2bf(v[3]) << 16);
        *reinterpret_cast<uint2*>(dst + 16 * dt) = w;
        __builtin_amdgcn_sched_barrier(0);
      }
      if (gl == 0) a.lse[lse_index(r)] = lse_nat;
    } else {
      uint16_t* dst = a.part_o + ((int64_t)s * a.R + r) * kDv + 4 * gl;
#pragma unroll
      for (int dt = 0; dt < kDv / 16; ++dt) {
        const f32x4 v = orow[dt] * scale;
        uint2 w;
        w.x = (uint32_t)f2bf(v[0]) | ((uint32_t)f2bf(v[1]) << 16);
        w.y = (uint32_t)f2bf(v[2]) | ((uint32_t)f2bf(v[3]) << 16);
        *reinterpret_cast<uint2*>(dst + 16 * dt) = w;
        __builtin_amdgcn_sched_barrier(0);
      }
      if (gl == 0) a.part_lse[(int64_t)s * a.R + r] = lse_nat;
    }
  }

  // LSE (natural log) and output scale of a row; the sink is folded in for final outputs.
  __device__ __forceinline__ void row_norm(int r, float m2, float l, bool final_out, float* lse_nat,
                                           float* scale) const {
    const float kLn2 = 0.69314718055994530942f;
    if (l > 0.f) {
      float lse = (m2 + __log2f(l)) * kLn2;
      float sc = 1.f / l;
      if (final_out && a.sink != nullptr) {
        const float sk = a.sink[head_of(r)];
        const float mx = fmaxf(lse, sk);
        const float lse2 = mx + __logf(__expf(lse - mx) + __expf(sk - mx));
        sc *= __expf(lse - lse2);
        lse = lse2;
      }
      *lse_nat = lse;
      *scale = sc;
    } else {
      *scale = 0.f;
      *lse_nat = (final_out && a.sink != nullptr) ? a.sink[head_of(r)] : kNegInf;
    }
  }

  __device__ __forceinline__ int head_of(int r) const { return (a.topk > 0) ? r : r % a.H; }
  __device__ __forceinline__ int64_t lse_index(int r) const {
    int bb, t, h;
    if (a.topk > 0) {
      bb = g / a.Sq;
      t = g % a.Sq;
      h = r;
    } else {
      bb = g;
      t = r / a.H;
      h = r % a.H;
    }
    return ((int64_t)bb * a.H + h) * a.Sq + t;
  }
};



// MFMAs with pinned register classes. The compiler keeps accumulators of builtin MFMAs in AGPRs
// but loop-carried values in VGPRs, copying every accumulator once per iteration; pinning S^T to
// VGPRs ("v") and O^T to AGPRs ("a") removes those copies. The hazard recogniser does not see
// inside inline asm, so every VALU read of their results goes through mfma_drain first.
__device__ __forceinline__ void mfma_s(f32x4& c, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(c) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_s0(f32x4& c, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, 0" : "=&v"(c) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_o(f32x4& c, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_o0(f32x4& c, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, 0" : "=&a"(c) : "v"(a), "v"(b));
}
// The last k step of a 2 x 2 block of S^T tiles: its four MFMAs and the wait for their results
// (19 wait states: more than an XDL write -> VALU read of a 16x16x32 result needs) in one statement. With the wait in a statement of its own, the compiler may place a copy of an
// accumulator (a register move it inserts for the tied operands) between the MFMA and the wait,
// where it would read the value before the MFMA has written it.
__device__ __forceinline__ void mfma_s_last4(f32x4& c00, f32x4& c01, f32x4& c10, f32x4& c11,
                                             const bf16x8& k0, const bf16x8& k1, const bf16x8& q0,
                                             const bf16x8& q1) {
  asm volatile(
      "v_mfma_f32_16x16x32_bf16 %0, %4, %6, %0\n\t"
      "v_mfma_f32_16x16x32_bf16 %1, %4, %7, %1\n\t"
      "v_mfma_f32_16x16x32_bf16 %2, %5, %6, %2\n\t"
      "v_mfma_f32_16x16x32_bf16 %3, %5, %7, %3\n\t"
      "s_nop 7\n\ts_nop 7\n\ts_nop 2"
      : "+v"(c00), "+v"(c01), "+v"(c10), "+v"(c11)
      : "v"(k0), "v"(k1), "v"(q0), "v"(q1));
}
// Score MFMAs with the Q^T operand held in accumulation registers.
__device__ __forceinline__ void mfma_sq(f32x4& c, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(c) : "v"(a), "a"(b));
}
__device__ __forceinline__ void mfma_sq0(f32x4& c, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, 0" : "=&v"(c) : "v"(a), "a"(b));
}
__device__ __forceinline__ void mfma_sq_last2(f32x4& c0, f32x4& c1, const bf16x8& a0,
                                              const bf16x8& a1, const bf16x8& b) {
  asm volatile(
      "v_mfma_f32_16x16x32_bf16 %0, %2, %4, %0\n\t"
      "v_mfma_f32_16x16x32_bf16 %1, %3, %4, %1\n\t"
      "s_nop 7\n\ts_nop 7\n\ts_nop 2"
      : "+v"(c0), "+v"(c1)
      : "v"(a0), "v"(a1), "a"(b));
}
// MFMAs whose operands were just written by VALU instructions (fp8 -> bf16 conversions): a VALU
// write of a VGPR needs two wait states before an MFMA reads it, which the compiler does not insert
// for inline assembly. Each statement waits three and takes every converted operand as an input.
__device__ __forceinline__ void mfma_sq2_cvt0(f32x4& c0, f32x4& c1, const bf16x8& a0, const bf16x8& a1,
                                              const bf16x8& b) {
  asm volatile(
      "s_nop 2\n\t"
      "v_mfma_f32_16x16x32_bf16 %0, %2, %4, 0\n\t"
      "v_mfma_f32_16x16x32_bf16 %1, %3, %4, 0"
      : "=&v"(c0), "=&v"(c1)
      : "v"(a0), "v"(a1), "a"(b));
}
__device__ __forceinline__ void mfma_sq2_cvt(f32x4& c0, f32x4& c1, const bf16x8& a0, const bf16x8& a1,
                                             const bf16x8& b) {
  asm volatile(
      "s_nop 2\n\t"
      "v_mfma_f32_16x16x32_bf16 %0, %2, %4, %0\n\t"
      "v_mfma_f32_16x16x32_bf16 %1, %3, %4, %1"
      : "+v"(c0), "+v"(c1)
      : "v"(a0), "v"(a1), "a"(b));
}
__device__ __forceinline__ void mfma_sq2_cvt_last(f32x4& c0, f32x4& c1, const bf16x8& a0,
                                                  const bf16x8& a1, const bf16x8& b) {
  asm volatile(
      "s_nop 2\n\t"
      "v_mfma_f32_16x16x32_bf16 %0, %2, %4, %0\n\t"
      "v_mfma_f32_16x16x32_bf16 %1, %3, %4, %1\n\t"
      "s_nop 7\n\ts_nop 7\n\ts_nop 2"
      : "+v"(c0), "+v"(c1)
      : "v"(a0), "v"(a1), "a"(b));
}
// An accumulator tile read into VGPRs by explicit copies: the tile stays an accumulation-register
// value for the compiler (a plain VALU use would make it re-home the whole array).
__device__ __forceinline__ f32x4 acc_read(const f32x4& o) {
  f32x4 v;
  asm volatile("v_accvgpr_read_b32 %0, %4\n\tv_accvgpr_read_b32 %1, %5\n\tv_accvgpr_read_b32 %2, %6\n\tv_accvgpr_read_b32 %3, %7"
               : "=v"(v[0]), "=v"(v[1]), "=v"(v[2]), "=v"(v[3])
               : "a"(o[0]), "a"(o[1]), "a"(o[2]), "a"(o[3]));
  return v;
}
template <int N, int M>
__device__ __forceinline__ void mfma_drain_acc(f32x4 (&o)[N][M]) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 2" ::: "memory");
#pragma unroll
  for (int i = 0; i < N; ++i)
#pragma unroll
    for (int k = 0; k < M; ++k) asm volatile("" : "+a"(o[i][k]));
}

// 64 query rows per workgroup, eight waves in two roles, two waves per SIMD:
//  * score waves 0-3: QK^T and the softmax of rows [16w, 16w + 16) of the tile (Q^T held in
//    accumulation registers), P^T handed to the value waves through a double-buffered LDS tile;
//  * value waves 4-7: O^T for output columns [128v, 128v + 128) of all 64 rows, plus every
//    global -> LDS transfer.
// In step t the score waves work on KV step t while the value waves accumulate step t - 1, so each
// SIMD interleaves one wave's MFMAs with the other's softmax, LDS waits and DMA issue. One
// workgroup barrier per step hands P^T over and recycles KV slots.
//
// KV rows stream through a ring of four 32-row LDS slots (K of step t and V of step t - 1 being
// read, steps t + 1 and t + 2 in flight). Value wave v moves rows [8v, 8v + 8) of every step. Step
// x's bundle, issued at the start of step x - 2, holds the LDS-DMA of step x's rows (zero-row reads
// past the split's end), the block-table entries of step x + 3 and, with index lists, the index
// entries of step x + 6. Block-table and index entries travel by LDS-DMA into small per-wave rings,
// so no register waits on an in-flight load; their addresses are clamped and the values validated
// when consumed. Every bundle holds the same number of memory operations, so "bundle x has landed"
// is an exact vmcnt.
template <int DQK, bool FP8>
struct Spec64 {
  // bf16 rows: latent region = the first 512 values (1056-byte LDS rows), RoPE region = values
  // 512..575 when present. fp8 rows: latent region = the kNope e4m3 bytes (512-byte LDS rows,
  // swizzled), RoPE region = the 64 bf16 tail values, then the eight ue8m0 scale bytes per row.
  static constexpr int kNope = DQK - 64;                   // fp8 values per row
  static constexpr bool HAS_B = FP8 || DQK > 512;          // RoPE region present
  static constexpr int KS = DQK / 32;                      // 32-wide k steps of QK^T
  static constexpr int KSN = FP8 ? kNope / 32 : 16;        // k steps read from the latent region
  static constexpr int kRopeSrc = FP8 ? kNope : 1024;      // byte offset of the RoPE tail in a row
  static constexpr int kRows = 32;                         // rows per slot / step
  static constexpr int kRowA = FP8 ? 512 : kRowStrideA;
  static constexpr int kSlotA = kRows * kRowA;
  static constexpr int kScOff = kSlotA + kRows * 128;      // fp8: scale bytes [32][8]
  static constexpr int kSlot = FP8 ? kScOff + kRows * 8 : kSlotA + (HAS_B ? kRows * 128 : 0);
  static_assert(kSlot % 256 == 0, "slot bases keep the low byte of in-slot offsets");
  static constexpr uint32_t kPOff = 4 * kSlot;             // P^T fragments [2][4 row tiles][64]
  static constexpr uint32_t kAOff = kPOff + 2 * 4096;      // rescale factors [2][64]
  static constexpr uint32_t kFOff = kAOff + 2 * 256;       // rescale flags [2][4]
  static constexpr uint32_t kMOff = kFOff + 32;            // row-valid masks [4 steps][4 bytes]
  static constexpr uint32_t kLOff = kMOff + 16;            // final l [64], then m [64]
  static constexpr uint32_t kRiOff = kLOff + 512;          // per value wave: block-table entries
  static constexpr int kRiWave = 4 * 32 + 8 * 32;          //   [4][8], index entries [8][8]
  // fp8 rows: V of a step dequantised to bf16 by the score waves (which convert those values for
  // QK^T anyway), [2 steps][32 rows][1056 B], read by the value waves as bf16 slots are
  static constexpr uint32_t kVOff = (kRiOff + 4 * kRiWave + 255) / 256 * 256;
  static constexpr uint32_t kVBuf = kRows * kRowStrideA;
  static constexpr int LDS = FP8 ? kVOff + 2 * kVBuf : kRiOff + 4 * kRiWave;
  static_assert(LDS <= 160 * 1024, "LDS of one workgroup");
  static constexpr int kDmaOps = FP8 ? 6 : 8 + (HAS_B ? 1 : 0);  // row LDS-DMA instructions per bundle

  const DecodeArgs& a;
  lds_ptr sm;
  int lane, wave;
  int g, b, L, j0, n, q0, qend, nsplit, cur_split;

  __device__ Spec64(const DecodeArgs& args, lds_ptr base) : a(args), sm(base) {
    lane = threadIdx.x & 63;
    wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  }

  // ===== value waves: row description pipeline and DMA =======================================
  // Value wave v describes rows 8v + (lane & 7) of a step (lanes 8..63 repeat lanes 0..7).
  __device__ __forceinline__ int vrow() const { return 8 * (wave - 4) + (lane & 7); }
  __device__ __forceinline__ uint32_t pg_slot(int x) const {
    return kRiOff + (wave - 4) * kRiWave + (x & 3) * 32;
  }
  __device__ __forceinline__ uint32_t ix_slot(int x) const {
    return kRiOff + (wave - 4) * kRiWave + 128 + (x & 7) * 32;
  }
  __device__ __forceinline__ void dma_dword(const int32_t* src, uint32_t dst) const {
    if (lane < 8)
      dma_x1(src, lds_addr(sm + dst));
  }
  __device__ __forceinline__ int ri_read(uint32_t slot) const {
    return *reinterpret_cast<const LDS_AS int*>(sm + slot + 4 * (lane & 7));
  }
  __device__ __forceinline__ void idx_fetch(int x) const {  // index entries of step x
    const int k = min(32 * x + vrow(), a.topk - 1);
    dma_dword(a.indices + (int64_t)g * a.topk + max(k, 0), ix_slot(x));
  }
  __device__ __forceinline__ int row_j(int x) const {  // logical position of the row
    return (a.topk > 0) ? ri_read(ix_slot(x)) : j0 + 32 * x + vrow();
  }
  __device__ __forceinline__ void page_fetch(int x) const {  // block-table entries of step x
    const int j = row_j(x);
    const int pi = min(max(j >> a.ps_log2, 0), a.max_pages - 1);
    dma_dword(a.block_table + (int64_t)b * a.max_pages + pi, pg_slot(x));
  }
  // Global address of the row (and, for fp8 rows, of its scale slot); invalid rows read the zero row.
  __device__ __forceinline__ uint64_t row_base(int x, bool* valid, uint64_t* scale_base) const {
    const int j = row_j(x);
    const int page = ri_read(pg_slot(x));
    const int k = 32 * x + vrow();
    bool ok = x < qend && k < n && (j >> a.ps_log2) < a.max_pages;
    if (a.topk > 0) ok = ok && j >= 0 && j < L;
    ok = ok && page >= 0 && (int64_t)page < a.num_pages;
    *valid = ok;
    if (!ok) {
      *scale_base = (uint64_t)(uintptr_t)a.zero_row;
      return (uint64_t)(uintptr_t)a.zero_row;
    }
    const int slot = j & ((1 << a.ps_log2) - 1);
    const uint8_t* pg = a.cache + (int64_t)page * a.page_stride;
    *scale_base = (uint64_t)(uintptr_t)(pg + a.scale_off + 8 * slot);
    return (uint64_t)(uintptr_t)(pg + (int64_t)slot * a.row_bytes);
  }
  __device__ __forceinline__ void bundle(int x) const {
    bool v;
    uint64_t sbase;
    const uint64_t base = row_base(x, &v, &sbase);
    const uint32_t m = (uint32_t)__ballot(v) & 0xFFu;
    if (lane == 0) *reinterpret_cast<LDS_AS uint8_t*>(sm + kMOff + 4 * (x & 3) + (wave - 4)) = (uint8_t)m;
    const uint32_t sa = (x & 3) * kSlot;
    const int r0 = 8 * (wave - 4);
    if constexpr (FP8) {
      // latent bytes: two 512-byte rows per instruction, chunks swizzled by row
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint64_t b0 = readlane64(base, 2 * i), b1 = readlane64(base, 2 * i + 1);
        const uint64_t rb = (lane < 32) ? b0 : b1;
        const int row = r0 + 2 * i + (lane >> 5);
        const uint8_t* src = reinterpret_cast<const uint8_t*>((uintptr_t)rb) + 16 * ((lane & 31) ^ swz_n(row));
        dma_x4(src, lds_addr(sm + sa + (r0 + 2 * i) * 512));
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i)
        dma_x4s(16 * lane, readlane64(base, i), lds_addr(sm + sa + (r0 + i) * kRowStrideA));
    }
    if constexpr (HAS_B) {
      const int r = r0 + (lane >> 3);
      const int c = (lane & 7) ^ swz_b(r);
      const uint32_t lo = __shfl((uint32_t)base, lane >> 3, 64);
      const uint32_t hi = __shfl((uint32_t)(base >> 32), lane >> 3, 64);
      const uint8_t* src = reinterpret_cast<const uint8_t*>((uintptr_t)(((uint64_t)hi << 32) | lo)) +
                           kRopeSrc + 16 * c;
      dma_x4(src, lds_addr(sm + sa + kSlotA + (wave - 4) * 1024));
    }
    if constexpr (FP8) {
      // scale slots: 8 rows x 8 bytes, one dword per lane
      const int sl = (lane >> 1) & 7;
      const uint32_t lo = __shfl((uint32_t)sbase, sl, 64);
      const uint32_t hi = __shfl((uint32_t)(sbase >> 32), sl, 64);
      // scale slots are 8-byte aligned: the dword offset is an OR into the low word
      const int32_t* src = reinterpret_cast<const int32_t*>((uintptr_t)(((uint64_t)hi << 32) | (lo | (4u * (lane & 1)))));
      if (lane < 16)
        dma_x1(src, lds_addr(sm + sa + kScOff + r0 * 8));
    }
    page_fetch(x + 3);
    if (a.topk > 0) idx_fetch(x + 6);
  }

  __device__ __forceinline__ void load_split(int s) {
    cur_split = s;
    // the split's descriptor (group, request, first row, rows, request length, step range, the
    // group's split count), kept in scalar registers (uniform across the workgroup)
    const int32_t* d = a.plan + a.sdesc_off + 8 * (int64_t)s;
    g = __builtin_amdgcn_readfirstlane(d[0]);
    b = __builtin_amdgcn_readfirstlane(d[1]);
    j0 = __builtin_amdgcn_readfirstlane(d[2]);
    n = __builtin_amdgcn_readfirstlane(d[3]);
    L = __builtin_amdgcn_readfirstlane(d[4]);
    q0 = __builtin_amdgcn_readfirstlane(d[5]);
    qend = __builtin_amdgcn_readfirstlane(d[6]);  // steps holding at least one row
    nsplit = __builtin_amdgcn_readfirstlane(d[7]);
  }

  // ===== score waves ===========================================================================
  __device__ void score_split(int mt) {
    const int nl = lane & 15, gl = lane >> 4;
    const int qrow = mt * 64 + wave * 16 + nl;  // this lane's softmax row
    // Q^T of the wave's 16 rows (rows past R repeat the last row; their outputs are dropped),
    // kept in accumulation registers for the whole split
    bf16x8 qr[KS];
    {
      const int r = min(qrow, a.R - 1);
      const bf16x8* src = reinterpret_cast<const bf16x8*>(a.q + ((int64_t)g * a.R + r) * DQK + 8 * gl);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) qr[ks] = src[4 * ks];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) asm volatile("" : "+a"(qr[ks]));
    }
    const bool sparse = a.topk > 0;
    const int qpos = L - a.Sq + (sparse ? 0 : (qrow / a.H));
    const bool dense_mask = !sparse && (a.causal || a.window > 0);
    float m_ref = kNegInf, l_acc = 0.f;
    float m_top = kNegInf;  // the row's true maximum (m_ref trails it by up to kTau)
    lds_barrier();  // prologue: step q0 landed

    for (int t = q0; t <= qend; ++t) {
      if (t < qend) {
        const uint32_t sa = (t & 3) * kSlot;
        const uint32_t sb = sa + kSlotA;
        // ---- S^T = K Q^T: 32 step rows x this wave's 16 rows -------------------------------
        uint32_t kaddr[2];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) kaddr[kt] = sa + (16 * kt + nl) * kRowStrideA + 16 * gl;
        // raw operand of k step ks: bf16 values, or (fp8 latent steps) eight e4m3 bytes
        auto k_raw = [&](int kt, int ks) -> bf16x8 {
          const int row = 16 * kt + nl;
          if (ks < KSN) {
            if constexpr (FP8) {
              const uint32_t ad = sa + row * 512 + 16 * ((2 * ks + (gl >> 1)) ^ swz_n(row)) + 8 * (gl & 1);
              const u32x2 w = *reinterpret_cast<const LDS_AS u32x2*>(sm + ad);
              return __builtin_bit_cast(bf16x8, u32x4{w[0], w[1], 0u, 0u});
            } else {
              return lds_read_b128(sm, kaddr[kt] + 64 * ks);
            }
          }
          const int c = (4 * (ks - KSN) + gl) ^ swz_b(row);
          return lds_read_b128(sm, sb + row * 128 + 16 * c);
        };
        // fp8 rows: the scale bytes of the lane's two K rows
        u32x2 ksc[2] = {u32x2{0u, 0u}, u32x2{0u, 0u}};
        if constexpr (FP8) {
#pragma unroll
          for (int kt = 0; kt < 2; ++kt)
            ksc[kt] = *reinterpret_cast<const LDS_AS u32x2*>(sm + sa + kScOff + 8 * (16 * kt + nl));
        }
        auto k_operand = [&](const bf16x8& raw, int kt, int ks) -> bf16x8 {
          if constexpr (FP8) {
            if (ks < KSN) {
              const u32x4 w = __builtin_bit_cast(u32x4, raw);
              const int gi = ks >> 1;  // 64-value scale group
              const uint32_t sw = (gi < 4) ? ksc[kt][0] : ksc[kt][1];
              return fp8x8_scaled(w[0], w[1], ue8m0_f32((sw >> (8 * (gi & 3))) & 0xFFu));
            }
          }
          return raw;
        };
        constexpr int D = 2;  // operand steps in flight
        bf16x8 ka[D][2];
#pragma unroll
        for (int i = 0; i < D - 1; ++i)
#pragma unroll
          for (int kt = 0; kt < 2; ++kt) ka[i][kt] = k_raw(kt, i);
        f32x4 sacc[2];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          if (ks + D - 1 < KS) {
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) ka[(ks + D - 1) % D][kt] = k_raw(kt, ks + D - 1);
          }
          const bf16x8 k0 = k_operand(ka[ks % D][0], 0, ks);
          const bf16x8 k1 = k_operand(ka[ks % D][1], 1, ks);
          if constexpr (FP8) {
            // the value columns of these operands, dequantised: score wave w stores k steps
            // ks = w mod 4 into the step's V tile
            if (32 * ks < kDv && (ks & 3) == wave) {
              const uint32_t vt = kVOff + (t & 1) * kVBuf + 2 * (32 * ks + 8 * gl);
              *reinterpret_cast<LDS_AS bf16x8*>(sm + vt + nl * kRowStrideA) = k0;
              *reinterpret_cast<LDS_AS bf16x8*>(sm + vt + (16 + nl) * kRowStrideA) = k1;
            }
            if (ks == KS - 1) mfma_sq2_cvt_last(sacc[0], sacc[1], k0, k1, qr[ks]);
            else if (ks == 0) mfma_sq2_cvt0(sacc[0], sacc[1], k0, k1, qr[0]);
            else mfma_sq2_cvt(sacc[0], sacc[1], k0, k1, qr[ks]);
          } else if (ks == KS - 1) {
            mfma_sq_last2(sacc[0], sacc[1], k0, k1, qr[ks]);
          } else if (ks == 0) {
            mfma_sq0(sacc[0], k0, qr[0]);
            mfma_sq0(sacc[1], k1, qr[0]);
          } else {
            mfma_sq(sacc[0], k0, qr[ks]);
            mfma_sq(sacc[1], k1, qr[ks]);
          }
        }

        // ---- masks ---------------------------------------------------------------------------
        const bool tail = 32 * (t + 1) > n;
        const uint32_t vmask = *reinterpret_cast<const LDS_AS uint32_t*>(sm + kMOff + 4 * (t & 3));
        const bool need_mask = sparse ? (vmask != ~0u) : (tail || dense_mask);
        if (need_mask) {
          const int causal_hi = a.causal ? 0 : (1 << 30);
          const int win = a.window > 0 ? a.window : (1 << 30);
#pragma unroll
          for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int row = 16 * kt + 4 * gl + e;
              const int k = 32 * t + row;
              const int j = j0 + k;
              const bool ok = sparse ? (((vmask >> row) & 1u) != 0)
                                     : (k < n && j <= qpos + causal_hi && j >= qpos - win + 1);
              sacc[kt][e] = ok ? sacc[kt][e] : kNegInf;
            }
        }

        // ---- softmax of this wave's rows (base 2, lazy reference maximum) --------------------
        float mx = kNegInf;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int e = 0; e < 4; ++e) mx = fmaxf(mx, sacc[kt][e]);
        mx = rows_max(mx);
        const float mnew = mx * a.scale_log2;  // -inf stays -inf (scale > 0)
        m_top = fmaxf(m_top, mnew);
        const bool up = mnew > m_ref + kTau;
        float alpha = 1.f;
        if (up) {
          alpha = __builtin_amdgcn_exp2f(m_ref - mnew);  // m_ref = -inf -> 0
          m_ref = mnew;
          l_acc *= alpha;
        }
        const float mu = (m_ref == kNegInf) ? 0.f : m_ref;
        bf16x8 pf;
        float lsum = 0.f;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kt][e], a.scale_log2, -mu));
            lsum += pv;
            pf[kt * 4 + e] = (__bf16)pv;
          }
        l_acc += lsum;
        const bool wave_up = __any(up);
        const uint32_t pb = (t & 1);
        *reinterpret_cast<LDS_AS bf16x8*>(sm + kPOff + pb * 4096 + (wave * 64 + lane) * 16) = pf;
        if (gl == 0) *reinterpret_cast<LDS_AS float*>(sm + kAOff + pb * 256 + 4 * (16 * wave + nl)) = alpha;
        if (lane == 0) *reinterpret_cast<LDS_AS int*>(sm + kFOff + pb * 16 + 4 * wave) = wave_up ? 1 : 0;
      }
      lds_barrier();  // P^T of step t published; K slot of step t released
    }
    // ---- row statistics for the value waves --------------------------------------------------
    const float lt = rows_sum(l_acc);
    if (gl == 0) {
      *reinterpret_cast<LDS_AS float*>(sm + kLOff + 4 * (wave * 16 + nl)) = lt;
      *reinterpret_cast<LDS_AS float*>(sm + kLOff + 256 + 4 * (wave * 16 + nl)) = m_ref;
      if (a.max_logits != nullptr && qrow < a.R) {  // natural-log units of the scaled scores
        const float ml = m_top * 0.69314718055994530942f;
        if (nsplit == 1) a.max_logits[lse_index(qrow)] = ml;
        else a.part_max[(int64_t)cur_split * a.R + qrow] = ml;
      }
    }
    lds_barrier();  // statistics published
    lds_barrier();  // output rows staged
    store_rows(mt);
    lds_barrier();  // staging area and slots reused by the next split
  }

  // Output rows of the tile leave LDS as whole 1 KB rows: wave w stores rows [8w, 8w + 8).
  static constexpr int kStageRow = 1040;  // 16 bytes of padding spread the 8-byte staging writes
  static_assert(64 * kStageRow <= 4 * kSlot, "output staging fits in the slots");
  __device__ __forceinline__ void store_rows(int mt) {
    const int s = cur_split;
    const bool final_out = (nsplit == 1);
#pragma unroll
    for (int rr = 0; rr < 8; ++rr) {
      const int hrow = 8 * wave + rr;
      const int r = mt * 64 + hrow;
      if (r < a.R) {
        const u32x4 v = *reinterpret_cast<const LDS_AS u32x4*>(sm + hrow * kStageRow + 16 * lane);
        uint16_t* dst = final_out ? a.out + ((int64_t)g * a.R + r) * kDv : a.part_o + ((int64_t)s * a.R + r) * kDv;
        st_global_b128(dst + 8 * lane, v);
      }
    }
  }

  // ===== value waves ===========================================================================
  __device__ void value_split(int s, int mt) {
    const int vw = wave - 4;
    const int nl = lane & 15, gl = lane >> 4;
    const bool sparse = a.topk > 0;
    f32x4 o[8][4];  // [output column tile of this wave][row tile]
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
#pragma unroll
      for (int ht = 0; ht < 4; ++ht) o[dt][ht] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
      asm volatile("" : "+a"(o[dt][0]), "+a"(o[dt][1]), "+a"(o[dt][2]), "+a"(o[dt][3]));

    // ---- prologue: row entries of the first steps, then bundles q0 and q0 + 1 ---------------
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // rings free
    if (sparse) {
#pragma unroll
      for (int i = 0; i < 6; ++i) idx_fetch(q0 + i);
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
#pragma unroll
    for (int i = 0; i < 3; ++i) page_fetch(q0 + i);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    bundle(q0);
    bundle(q0 + 1);
    // bundle q0 landed, bundle q0 + 1 may be in flight
    if (sparse) asm volatile("s_waitcnt vmcnt(%0)" :: "n"(kDmaOps + 2) : "memory");
    else asm volatile("s_waitcnt vmcnt(%0)" :: "n"(kDmaOps + 1) : "memory");
    lds_barrier();

    for (int t = q0; t <= qend; ++t) {
      // bundle t + 2 goes into the slot of step t - 2, released at the last barrier. bf16 rows issue
      // it first, so its issue overlaps the score waves' QK^T; fp8 rows issue it after PV, so that
      // no wait in the PV section (register reloads of the converting code) waits on it.
      if constexpr (!FP8) bundle(t + 2);
      if (t > q0) {
        const int u = t - 1;  // step accumulated now
        const uint32_t pbo = (u & 1);
        const LDS_AS int* fl = reinterpret_cast<const LDS_AS int*>(sm + kFOff + pbo * 16);
        const int f0 = fl[0], f1 = fl[1], f2 = fl[2], f3 = fl[3];
        if (f0 | f1 | f2 | f3) {
          // only the row tiles whose score wave moved its reference maximum (tile ht = wave ht)
          mfma_drain_acc(o);
#pragma unroll
          for (int ht = 0; ht < 4; ++ht) {
            const int f = (ht == 0) ? f0 : (ht == 1) ? f1 : (ht == 2) ? f2 : f3;
            if (!f) continue;
            const float al = *reinterpret_cast<const LDS_AS float*>(sm + kAOff + pbo * 256 + 4 * (16 * ht + nl));
#pragma unroll
            for (int dt = 0; dt < 8; ++dt) {
              o[dt][ht] *= al;
              asm volatile("" : "+a"(o[dt][ht]));  // back to its accumulation registers now
              __builtin_amdgcn_sched_barrier(0);
            }
          }
        }
        bf16x8 pb[4];
#pragma unroll
        for (int ht = 0; ht < 4; ++ht)
          pb[ht] = *reinterpret_cast<const LDS_AS bf16x8*>(sm + kPOff + pbo * 4096 + (ht * 64 + lane) * 16);
        const uint32_t su = (u & 3) * kSlot;
        // V^T operand rows: k slot 8 gl + e holds KV row 4 gl + e (e < 4) or 12 + 4 gl + e, the
        // order of the P^T fragments
        __builtin_assume(vw >= 0 && vw < 4);
        // fp8 rows: scale bytes of the lane's eight KV rows, for the wave's two column groups
        // (group 2 vw for tiles 0..3, 2 vw + 1 for tiles 4..7), read as needed
        // V^T operand of output tile dt: bf16 rows of the step's slot, or for fp8 rows of its V
        // tile (dequantised by the score waves in step u)
        const uint32_t vbase = FP8 ? kVOff + (u & 1) * kVBuf : su;
        auto v_raw = [&](int dt) -> bf16x8 {
          const int col0 = 128 * vw + 16 * dt;  // first output column of the tile
          const uint32_t ad = vbase + (4 * gl + (nl >> 2)) * kRowStrideA + 8 * (lane & 3) + 2 * col0;
          const bf16x4 v0 = lds_read_tr(sm, ad);
          const bf16x4 v1 = lds_read_tr(sm, ad + 16 * kRowStrideA);
          return __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
        };
        // V operand tiles in flight
        constexpr int VD = 3;
        bf16x8 va[VD];
#pragma unroll
        for (int i = 0; i < VD - 1; ++i) va[i] = v_raw(i);
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
          if (dt + VD - 1 < 8) va[(dt + VD - 1) % VD] = v_raw(dt + VD - 1);
#pragma unroll
          for (int ht = 0; ht < 4; ++ht) mfma_o(o[dt][ht], va[dt % VD], pb[ht]);
        }
      }
      if constexpr (FP8) bundle(t + 2);
      // bundle t + 1 landed (K of the next step), bundle t + 2 may be in flight
      if (sparse) asm volatile("s_waitcnt vmcnt(%0)" :: "n"(kDmaOps + 2) : "memory");
      else asm volatile("s_waitcnt vmcnt(%0)" :: "n"(kDmaOps + 1) : "memory");
      lds_barrier();
    }
    // the last bundles (zero-row reads) must land before the slots are reused
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    mfma_drain_acc(o);
    lds_barrier();  // score waves' statistics published

    // ---- epilogue: each value wave normalises its 128 columns of all 64 rows into the staging
    // rows (all slots are free: every bundle landed before the last barrier) ------------------
    const bool final_out = (nsplit == 1);
    const int tile0 = mt * 64;
#pragma unroll
    for (int ht = 0; ht < 4; ++ht) {
      const int hrow = ht * 16 + nl;
      const int r = tile0 + hrow;
      const float lt = *reinterpret_cast<const LDS_AS float*>(sm + kLOff + 4 * hrow);
      const float m2 = *reinterpret_cast<const LDS_AS float*>(sm + kLOff + 256 + 4 * hrow);
      float lse_nat, scale;
      row_norm(min(r, a.R - 1), m2, lt, final_out, &lse_nat, &scale);
      const uint32_t row_at = hrow * kStageRow + 2 * (128 * vw + 4 * gl);
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        const f32x4 v = o[dt][ht] * scale;
        const u32x2 w = {(uint32_t)f2bf(v[0]) | ((uint32_t)f2bf(v[1]) << 16),
                         (uint32_t)f2bf(v[2]) | ((uint32_t)f2bf(v[3]) << 16)};
        *reinterpret_cast<LDS_AS u32x2*>(sm + row_at + 32 * dt) = w;
      }
      if (vw == 0 && gl == 0 && r < a.R) {
        if (final_out) a.lse[lse_index(r)] = lse_nat;
        else a.part_lse[(int64_t)s * a.R + r] = lse_nat;
      }
    }
    lds_barrier();  // output rows staged
    store_rows(mt);
    lds_barrier();  // staging area and slots reused by the next split
  }

  // LSE (natural log) and output scale of a row; the sink is folded in for final outputs.
  __device__ __forceinline__ void row_norm(int r, float m2, float l, bool final_out, float* lse_nat,
                                           float* scale) const {
    const float kLn2 = 0.69314718055994530942f;
    if (l > 0.f) {
      float lse = (m2 + __log2f(l)) * kLn2;
      float sc = 1.f / l;
      if (final_out && a.sink != nullptr) {
        const float sk = a.sink[(a.topk > 0) ? r : r % a.H];
        const float mx = fmaxf(lse, sk);
        const float lse2 = mx + __logf(__expf(lse - mx) + __expf(sk - mx));
        sc *= __expf(lse - lse2);
        lse = lse2;
      }
      *lse_nat = lse;
      *scale = sc;
    } else {
      *scale = 0.f;
      *lse_nat = (final_out && a.sink != nullptr) ? a.sink[(a.topk > 0) ? r : r % a.H] : kNegInf;
    }
  }
  __device__ __forceinline__ int64_t lse_index(int r) const {
    int bb, t, h;
    if (a.topk > 0) {
      bb = g / a.Sq;
      t = g % a.Sq;
      h = r;
    } else {
      bb = g;
      t = r / a.H;
      h = r % a.H;
    }
    return ((int64_t)bb * a.H + h) * a.Sq + t;
  }
};

// 128 query rows per workgroup for bf16 rows: all heads of a DeepSeek-V3 request, so every KV row
// enters one CU once. Four waves, one per SIMD, all in one role: wave w owns query rows
// [32w, 32w + 32) of the tile for a whole split. It holds their Q^T in registers, computes
// S^T = K Q^T, the softmax, and O^T += V^T P^T over all 512 output columns. Its 32 x 512 fp32
// accumulator lives in the 256 accumulation registers, and P^T never leaves the wave. The waves
// share only the KV rows in LDS, a ring of four 32-row slots, and one workgroup barrier per step.
//
// The step loop is software-pipelined so the MFMA pipe has work while the wave does everything
// else. Iteration k runs QK^T of step k with the softmax of step k - 1 spread between its MFMAs,
// and the row transfers of step k + 2 spread there too; then PV of step k - 1, with the row
// addresses of step k + 3 worked out between its MFMAs. Slots k - 1 and k are read in iteration k,
// k + 1 and k + 2 are landing; the barrier at the top of iteration k both publishes step k's rows
// and frees the slot of step k - 2 for step k + 2.
//
// A unit's splits are taken in chunks of up to kChunk, whose descriptors sit in LDS. Within a
// chunk the row stream runs on across split boundaries: a boundary costs the epilogue (the wave's
// rows normalised, staged through the slot just read and stored as whole 128-byte lines) and the
// load of the next split's Q^T, not a refill of the ring.
//
// Step y's bundle holds the LDS-DMA of its rows, the block-table entries of step y + 3 and, with
// index lists, the index entries of step y + 6. All three travel by LDS-DMA into small per-wave
// rings, so no register waits on an in-flight load; their addresses are clamped and their values
// validated when consumed. Bundles past the chunk's last step read the zero row, so every bundle
// holds the same number of memory instructions and "bundle k has landed" is always the same
// vmcnt (one later bundle in flight).
//
// fp8 rows (FP8, dense rows only): a bundle lands in a ring of three fp8 entries (e4m3 bytes, the
// bf16 RoPE tail and the ue8m0 scale bytes of its 32 rows) and is converted once into a bf16 slot
// of the layout above (latent values only; QK^T reads the RoPE tail from the ring entry, where its
// 16-byte chunks land swizzled as in a RoPE region). Each wave converts its own eight rows of step
// k + 1 between the PV MFMAs of iteration k, after waiting for its own transfers of that bundle, so
// the conversion runs in the MFMA pipe's shadow and the step keeps its one barrier. Three bf16
// slots (QK^T of step k, PV of step k - 1, conversion of step k + 1) and the ring fill the LDS; the
// block-table and index tables, which only index lists need, are left out.
template <int DQK, bool MAXL, bool SPARSE, bool FP8 = false>
struct Tile128 {
  static_assert(!FP8 || (!SPARSE && !MAXL), "fp8 rows: dense decode only");
  static constexpr bool HAS_B = DQK > 512;               // RoPE region present
  static constexpr int KS = DQK / 32;                    // 32-wide k steps of QK^T
  static constexpr int kRows = 32;                       // rows per slot / step
  static constexpr int NS = FP8 ? 3 : 4;                 // bf16 slots
  static constexpr int kSlotA = kRows * kRowStrideA;
  static constexpr int kSlot = kSlotA + ((HAS_B && !FP8) ? kRows * 128 : 0);
  static_assert(kSlot % 256 == 0, "slot bases keep the low byte of in-slot offsets");
  // fp8 ring entry: e4m3 bytes [32 rows][512] (kNope used), RoPE tails [32][128], scales [32][8]
  static constexpr int kNope = DQK - 64;
  static constexpr uint32_t kRingRope = kRows * 512;
  static constexpr uint32_t kRingSc = kRingRope + kRows * 128;
  static constexpr uint32_t kRingEntry = kRingSc + kRows * 8;
  static_assert(kRingEntry % 256 == 0, "ring entries keep the low byte of in-entry offsets");
  static constexpr int NR = 3;                           // fp8 ring entries
  static constexpr uint32_t kRingOff = NS * kSlot;
  // index lists only: block-table entries [4 waves][4 steps][8], index entries [4 waves][8 steps][8],
  // row-valid masks [8 steps][4 waves] bytes, the next bundle's row addresses [4 waves][8]
  static constexpr uint32_t kPgOff = kRingOff + (FP8 ? NR * kRingEntry : 0);
  static constexpr uint32_t kIxOff = kPgOff + (SPARSE ? 4 * 4 * 32 : 0);
  static constexpr uint32_t kMOff = kIxOff + (SPARSE ? 4 * 8 * 32 : 0);
  static constexpr uint32_t kDOff = kMOff + (SPARSE ? 32 : 0);  // split descriptors [kChunk][8 words]
  static constexpr int kChunk = FP8 ? 8 : 16;
  static constexpr uint32_t kRbOff = kDOff + kChunk * 32;
  static constexpr int LDS = kRbOff + (SPARSE ? 4 * 64 : 0);
  static_assert(LDS <= 160 * 1024, "LDS of one workgroup");
  static constexpr int kStageRow = (HAS_B && !FP8) ? 544 : 528;  // epilogue staging: 256 columns + pad
  static_assert(4 * 16 * kStageRow <= kSlot, "epilogue staging fits in one slot");
  // memory instructions per bundle: 8 rows, the RoPE tails (+ with index lists the block-table and
  // index dwords); fp8 rows: 4 transfers of two rows' e4m3 bytes, the RoPE tails, the scale bytes
  static constexpr int kNb = FP8 ? 6 : 8 + (HAS_B ? 1 : 0) + (SPARSE ? 2 : 0);
  // LDS offsets of bf16 slot x and fp8 ring entry x
  __device__ __forceinline__ static uint32_t slot_off(int x) {
    return (uint32_t)(NS == 4 ? (x & 3) : (x % NS)) * (uint32_t)kSlot;
  }
  __device__ __forceinline__ static uint32_t ring_off(int x) { return kRingOff + (uint32_t)(x % NR) * kRingEntry; }
  static constexpr bool sparse = SPARSE;
  enum { D_G, D_B, D_J0, D_N, D_L, D_Q0, D_QEND, D_NSPLIT };

  // A position in the chunk's step stream: step t of split ci (ci == nc: past the chunk's end).
  struct Cur {
    int y;     // step index in the chunk's stream
    int ci;    // split within the chunk
    int t;     // step within the split
    int q0, qend;        // the split's step range
    int g, b, j0, n, L;  // the split's group, request, first row, row count, request length
  };
  // Dense rows of a bundle: the wave's eight rows are consecutive positions j .. j + 7, on at most
  // two pages, whose block-table entries e0 (page of j) and e1 (page of j + 7) come through the
  // scalar cache; k is the rows' offset in the group, n the group's row count. Wave-uniform.
  struct DRows {
    int e0, e1, j, k, n;
  };
  // The bundle's row addresses in closed form: rows i < isplit lie on page e0 (b0 + i row_bytes),
  // the rest on page e1 (b1 + (i - isplit) row_bytes); rows i >= nvalid read the zero row.
  struct DAddr {
    uint64_t b0, b1;
    int isplit, nvalid;
    uint64_t s0, s1;  // fp8 rows: the scale slots of row 0 on page e0 and of the first row on e1
  };
  // Softmax state of the split whose step is being finished, and the step's own values.
  struct Soft {
    float m_ref[2], l_acc[2], m_top[2];  // per row tile: reference maximum, sum, true maximum
    float alpha[2], mu[2], lsum[2], mx[2], mnew[2], part[2];
    float sink[2];   // sink logits of the split's rows (-inf: none)
    bool up[2];
    bf16x8 pf[2];  // P^T of the step
  };
  // Lane constants, worked out once per chunk: the step loop issues one wave's every instruction,
  // and a VALU instruction costs the step about as much as it takes to issue, so the per-lane
  // parts of the operand and transfer addresses are not recomputed each step.
  struct Lane {
    int ln;        // lane
    uint32_t v16;  // 16 * lane: the lane's byte offset in a 1 KB transfer
    uint32_t kr;   // K^T operand, RoPE region: nl * 128 + 16 (gl ^ swz_b(nl)) (chunk 4 + gl: ^ 64)
    uint32_t irb;  // RoPE transfer: row (lane >> 3) * row bytes + the lane's byte offset in that row
    uint32_t kq_;  // K^T operand (rows nl, nl + 16 of a slot): nl * row stride + 16 gl
    uint32_t vq_;  // V^T operand: row 4 gl + (nl >> 2) = lane >> 2, column 4 (nl & 3)
    __device__ __forceinline__ uint32_t kq() const { return kq_; }
    __device__ __forceinline__ uint32_t vq() const { return vq_; }
    __device__ __forceinline__ int i2() const { return ln >> 3; }
    __device__ __forceinline__ uint32_t c16() const { return v16 ^ (uint32_t)(128 * (ln >> 5)) ^ (v16 & 512u); }
  };
  __device__ __forceinline__ Lane make_lane() const {
    Lane L;
    L.ln = lane_id();
    L.v16 = 16u * (uint32_t)L.ln;
    const int nl = L.ln & 15, gl = L.ln >> 4;
    L.kr = (uint32_t)(nl * 128 + 16 * (gl ^ swz_b(nl)));
    L.kq_ = (uint32_t)(nl * kRowStrideA + 16 * gl);
    L.vq_ = (uint32_t)((L.ln >> 2) * kRowStrideA + 8 * (L.ln & 3));
    const int i2 = L.ln >> 3;
    const int ch = (L.ln & 7) ^ ((HAS_B || !FP8) ? swz_b(8 * wave + i2) : 0);
    L.irb = (uint32_t)i2 * (uint32_t)a.row_bytes + (uint32_t)((FP8 ? kNope : 1024) + 16 * ch);
    return L;
  }

  const DecodeArgs& a;
  lds_ptr sm;
  int wave, mt;
  int num_pages32;  // page count, clamped to the int range (32-bit compares stay scalar)
  int nc, T;  // splits and steps of the current chunk
  int tok_lo, tok_hi;  // dense rows: the first and last query token among the wave's rows

  __device__ Tile128(const DecodeArgs& args, lds_ptr base, int tile) : a(args), sm(base), mt(tile) {
    wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    num_pages32 = (int)min(a.num_pages, (int64_t)0x7fffffff);
    tok_lo = min(mt * 128 + 32 * wave, a.R - 1) / a.H;
    tok_hi = min(mt * 128 + 32 * wave + 31, a.R - 1) / a.H;
  }

  // The lane index, read from the hardware each time it is asked for: addresses derived from it
  // are recomputed where they are used instead of being held in registers (or spilled) for the
  // whole kernel.
  __device__ __forceinline__ int lane_id() const {
    int l;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
    return l;
  }
  __device__ __forceinline__ int desc(int ci, int f) const {
    return __builtin_amdgcn_readfirstlane(*reinterpret_cast<const LDS_AS int*>(sm + kDOff + 32 * ci + 4 * f));
  }
  __device__ __forceinline__ Cur cur_load(Cur c) const {
    c.q0 = desc(c.ci, D_Q0);
    c.t = c.q0;
    c.qend = desc(c.ci, D_QEND);
    c.g = desc(c.ci, D_G);
    c.b = desc(c.ci, D_B);
    c.j0 = desc(c.ci, D_J0);
    c.n = desc(c.ci, D_N);
    c.L = desc(c.ci, D_L);
    return c;
  }
  __device__ __forceinline__ Cur cur_begin() const {
    Cur c;
    c.y = 0;
    c.ci = 0;
    return cur_load(c);
  }
  // the step after c
  __device__ __forceinline__ Cur cur_next(Cur c) const {
    ++c.y;
    if (++c.t >= c.qend) {
      if (++c.ci < nc) {
        c = cur_load(c);
      } else {  // past the chunk: every row invalid
        c.ci = nc;
        c.t = 0;
        c.q0 = 0;
        c.qend = 1 << 30;
        c.n = 0;
      }
    }
    return c;
  }

  // ===== descriptors of a chunk ===============================================================
  // Lane i of wave 0 describes split cb + i: its group, request, first row and row count, the
  // request's length, its step range and the group's split count.
  __device__ void build_table(int cb) {
    const int ln = lane_id();
    if (wave == 0 && ln < nc) {
      const int s = cb + ln;
      // the plan's descriptor of the split, in the order of the D_ fields
      const u32x4* src = reinterpret_cast<const u32x4*>(a.plan + a.sdesc_off + 8 * (int64_t)s);
      const u32x4 v0 = src[0], v1 = src[1];
      LDS_AS u32x4* d = reinterpret_cast<LDS_AS u32x4*>(sm + kDOff + 32 * ln);
      d[0] = v0;
      d[1] = v1;
    }
  }

  // ===== row transfers =========================================================================
  // Row i (0-7) of the wave's eight rows of a step is row 8w + i of the step.
  __device__ __forceinline__ uint32_t pg_slot(int y) const { return kPgOff + wave * 128 + (y & 3) * 32; }
  __device__ __forceinline__ uint32_t ix_slot(int y) const { return kIxOff + wave * 256 + (y & 7) * 32; }
  __device__ __forceinline__ int ring_read(uint32_t slot, int i) const {
    return *reinterpret_cast<const LDS_AS int*>(sm + slot + 4 * i);
  }
  // position of row i of step c (dense: from the cursor; index lists: the index entry in LDS)
  __device__ __forceinline__ int row_j(Cur c, int i) const {
    return sparse ? ring_read(ix_slot(c.y), i) : c.j0 + kRows * c.t + 8 * wave + i;
  }
  __device__ __forceinline__ const int32_t* idx_src(Cur c) const {
    const int k = min(kRows * c.t + 8 * wave + (lane_id() & 7), a.topk - 1);
    const int32_t* p = a.indices + (int64_t)c.g * a.topk + max(k, 0);
    return c.ci < nc ? p : reinterpret_cast<const int32_t*>(a.zero_row);
  }
  __device__ __forceinline__ const int32_t* page_src(Cur c) const {
    const int pi = min(max(row_j(c, lane_id() & 7) >> a.ps_log2, 0), a.max_pages - 1);
    const int32_t* p = a.block_table + (int64_t)c.b * a.max_pages + pi;
    return c.ci < nc ? p : reinterpret_cast<const int32_t*>(a.zero_row);
  }
  // Block-table or index entries of one step (lanes 0-7, one dword each).
  __device__ __forceinline__ void dma_dword(const int32_t* src, uint32_t dst) const {
    if (lane_id() < 8) dma_x1(src, lds_addr(sm + dst));
  }
  // Block-table entries of dense bundle c, loaded a step before its transfers.
  __device__ __forceinline__ DRows dense_rows(Cur c) const {
    DRows d;
    d.k = kRows * c.t + 8 * wave;
    d.j = c.j0 + d.k;
    d.n = c.n;  // 0 past the chunk: every row invalid
    const int p0 = min(max(d.j >> a.ps_log2, 0), a.max_pages - 1);
    const int p1 = min(max((d.j + 7) >> a.ps_log2, 0), a.max_pages - 1);
    typedef const __attribute__((address_space(4))) int32_t* const_i32p;  // scalar loads
    const const_i32p bt = (const_i32p)(uintptr_t)a.block_table + (int64_t)c.b * a.max_pages;
    d.e0 = bt[p0];
    d.e1 = bt[p1];
    return d;
  }
  __device__ __forceinline__ uint64_t page_base(int e, uint32_t slot) const {
    const bool ok = (e >= 0) & (e < num_pages32);
    const uint64_t addr = (uint64_t)(uintptr_t)a.cache + (uint64_t)(uint32_t)e * (uint64_t)(uint32_t)a.page_stride +
                          (uint64_t)(slot * (uint32_t)a.row_bytes);
    return ok ? addr : (uint64_t)(uintptr_t)a.zero_row;
  }
  __device__ __forceinline__ uint64_t scale_base(int e, uint32_t slot) const {
    const bool ok = (e >= 0) & (e < num_pages32);
    const uint64_t addr = (uint64_t)(uintptr_t)a.cache + (uint64_t)(uint32_t)e * (uint64_t)(uint32_t)a.page_stride +
                          (uint64_t)a.scale_off + 8u * slot;
    return ok ? addr : (uint64_t)(uintptr_t)a.zero_row;
  }
  __device__ __forceinline__ DAddr dense_addr(const DRows& d) const {
    DAddr r;
    const int ps = 1 << a.ps_log2;
    const int in0 = d.j & (ps - 1);
    r.isplit = min(ps - in0, 8);
    const int e0 = (d.j >> a.ps_log2) < a.max_pages ? d.e0 : -1;
    const int e1 = ((d.j + 7) >> a.ps_log2) < a.max_pages ? d.e1 : -1;
    r.b0 = page_base(e0, (uint32_t)in0);
    r.b1 = page_base(e1, 0u);
    r.nvalid = min(max(d.n - d.k, 0), 8);
    if constexpr (FP8) {
      r.s0 = scale_base(e0, (uint32_t)in0);
      r.s1 = scale_base(e1, 0u);
    }
    return r;
  }
  // Scale slot of dense fp8 row i, or the zero row.
  __device__ __forceinline__ uint64_t drow_sc(const DAddr& r, int i) const {
    const uint64_t on0 = r.s0 + (uint64_t)(uint32_t)(8 * i);
    const uint64_t on1 = r.s1 + (uint64_t)(uint32_t)(8 * (i - r.isplit));
    const uint64_t addr = (i < r.isplit) ? on0 : on1;
    return (i < r.nvalid) ? addr : (uint64_t)(uintptr_t)a.zero_row;
  }
  // Address of dense row i (+ off), or of the zero row (+ off) when the row lies past the group's
  // rows or its page entry is out of range (then page_base gave the zero row).
  __device__ __forceinline__ uint64_t drow(const DAddr& r, int i, uint32_t off) const {
    const uint64_t on0 = r.b0 + (uint64_t)(uint32_t)(i * (int)a.row_bytes);
    const uint64_t on1 = r.b1 + (uint64_t)(uint32_t)((i - r.isplit) * (int)a.row_bytes);
    const uint64_t addr = (i < r.isplit) ? on0 : on1;
    return ((i < r.nvalid) ? addr : (uint64_t)(uintptr_t)a.zero_row) + off;
  }
  // The RoPE transfer's source for each lane: row L.i2 of the bundle + L.roff, or the zero row + L.roff.
  __device__ __forceinline__ uint64_t drow_lane(const DAddr& r, const Lane& L) const {
    if (r.isplit >= 8 && r.nvalid >= 8) return r.b0 + (uint64_t)L.irb;  // the usual case: one page, all valid
    const uint64_t b1m = r.b1 - (uint64_t)(uint32_t)(r.isplit * (int)a.row_bytes);  // b1m + i rb: row i >= isplit
    const int i2 = L.i2();
    const uint64_t base = (i2 < r.isplit) ? r.b0 : b1m;
    const uint64_t zero = (uint64_t)(uintptr_t)a.zero_row - (uint64_t)(uint32_t)((uint32_t)i2 * (uint32_t)a.row_bytes);
    return ((i2 < r.nvalid) ? base : zero) + (uint64_t)L.irb;
  }
  // Address of row i of step c, or the zero row (then *ok is false).
  __device__ __forceinline__ uint64_t row_addr(Cur c, int i, int j, int page, bool* ok) const {
    const int k = kRows * c.t + 8 * wave + i;
    bool v = k < c.n && (j >> a.ps_log2) < a.max_pages;
    if (sparse) v = v && j >= 0 && j < c.L;
    v = v && page >= 0 && (int64_t)page < a.num_pages;
    *ok = v;
    const uint32_t slot = (uint32_t)(j & ((1 << a.ps_log2) - 1));
    const uint64_t addr = (uint64_t)(uintptr_t)a.cache + (uint64_t)(uint32_t)page * (uint64_t)(uint32_t)a.page_stride +
                          (uint64_t)(slot * (uint32_t)a.row_bytes);
    return v ? addr : (uint64_t)(uintptr_t)a.zero_row;
  }
  // Row addresses of bundle c (into the wave's table in LDS) and the row-valid mask of step c
  // (for its consumers): lanes 0-7 work out rows 0-7.
  __device__ __forceinline__ void prepare(Cur c, const Lane& L) const {
    const int ln = L.ln;
    const int i = ln & 7;
    const int pg = ring_read(pg_slot(c.y), i);
    const int j = row_j(c, i);
    bool ok;
    const uint64_t base = row_addr(c, i, j, pg, &ok);
    const uint32_t m = (uint32_t)__ballot(ok) & 0xFFu;
    if (ln == 0) *reinterpret_cast<LDS_AS uint8_t*>(sm + kMOff + 4 * (c.y & 7) + wave) = (uint8_t)m;
    if (ln < 8) *reinterpret_cast<LDS_AS uint64_t*>(sm + kRbOff + wave * 64 + 8 * i) = base;
  }
  __device__ __forceinline__ uint64_t rb_read(int i) const {  // row i's address (wave-uniform)
    return *reinterpret_cast<const LDS_AS uint64_t*>(sm + kRbOff + wave * 64 + 8 * i);
  }
  // Transfer s (0-10) of bundle y (page step cp = y + 3, index step cx = y + 6): rows 0-7 (row s's
  // address read one transfer ahead into `next`), the RoPE tails, then the ring entries.
  __device__ __forceinline__ void send_part(int s, int y, Cur cp, Cur cx, uint64_t& next, const DAddr& d,
                                           const Lane& L) const {
    if constexpr (FP8) {  // into ring entry y mod 3
      const uint32_t re = ring_off(y);
      const int ln = L.ln;
      if (s < 4) {  // e4m3 bytes of rows 2s and 2s + 1: lanes 0-31 and 32-63, chunks swizzled
        const uint32_t co = L.c16() ^ (16u * (uint32_t)s);
        uint64_t src;
        if (d.isplit >= 8 && d.nvalid >= 8) {  // the usual case: one page, all valid
          const uint32_t hr = (uint32_t)(ln >> 5) * (uint32_t)a.row_bytes;
          src = d.b0 + (uint64_t)(uint32_t)(2 * s * (int)a.row_bytes) + (uint64_t)(hr + co);
        } else {
          const uint64_t r0 = drow(d, 2 * s, 0), r1 = drow(d, 2 * s + 1, 0);
          src = (ln < 32 ? r0 : r1) + (uint64_t)co;
        }
        dma_x4<kRowsNT>(reinterpret_cast<const void*>((uintptr_t)src), lds_addr(sm + re + (8 * wave + 2 * s) * 512));
      } else if (s == 4) {  // RoPE tails: 16 bytes per lane, row ln >> 3 (chunks swizzled for QK^T)
        const uint64_t src = drow_lane(d, L);
        dma_x4<kRowsNT>(reinterpret_cast<const void*>((uintptr_t)src), lds_addr(sm + re + kRingRope + wave * 1024));
      } else if (s == 5) {  // scale bytes: one dword per lane, lanes 0-15
        const uint64_t src = drow_sc(d, (ln >> 1) & 7) + 4u * (uint32_t)(ln & 1);
        if (ln < 16) dma_x1(reinterpret_cast<const int32_t*>((uintptr_t)src), lds_addr(sm + re + kRingSc + wave * 64));
      }
      return;
    }
    const uint32_t sa = slot_off(y);
    if constexpr (!SPARSE) {  // dense: addresses from the scalar block-table entries
      if (s < 8) {
        dma_x4s<kRowsNT>(L.v16, drow(d, s, 0), lds_addr(sm + sa + (8 * wave + s) * kRowStrideA));
      } else if (s == 8) {
        if constexpr (HAS_B) {
          const uint64_t rope = drow_lane(d, L);
          dma_x4<kRowsNT>(reinterpret_cast<const void*>((uintptr_t)rope), lds_addr(sm + sa + kSlotA + wave * 1024));
        }
      }
      return;
    }
    if (s < 8) {
      const uint64_t row = readlane64(next, 0);
      if (s < 7) next = rb_read(s + 1);
      dma_x4s<kRowsNT>(L.v16, row, lds_addr(sm + sa + (8 * wave + s) * kRowStrideA));
    } else if (s == 8) {
      if constexpr (HAS_B) {
        const int ln = L.ln;
        const int i2 = ln >> 3;
        const uint64_t rope = rb_read(i2) + 1024 + 16 * ((ln & 7) ^ swz_b(8 * wave + i2));
        dma_x4<kRowsNT>(reinterpret_cast<const void*>((uintptr_t)rope), lds_addr(sm + sa + kSlotA + wave * 1024));
      }
    } else if (s == 9) {
      dma_dword(page_src(cp), pg_slot(y + 3));
    } else if (s == 10) {
      if (sparse) dma_dword(idx_src(cx), ix_slot(y + 6));
    }
  }
  __device__ __forceinline__ void send_all(int y, Cur cp, Cur cx, const DAddr& d, const Lane& L) const {
    uint64_t next = SPARSE ? rb_read(0) : 0;
#pragma unroll
    for (int s = 0; s < (FP8 ? kNb : 11); ++s) send_part(s, y, cp, cx, next, d, L);
  }
  // fp8 ring rows: 16-byte chunk c of row r sits at chunk c ^ swz_ring(r), so each 16-lane quarter
  // of the conversion's reads (lanes: rows r .. r + 7, chunk 4 g + i of two groups g) covers all
  // LDS banks once.
  __device__ __forceinline__ static int swz_ring(int r) { return ((r & 1) << 3) | ((r >> 1) & 3); }
  // fp8 rows: bundle x from its ring entry into bf16 slot x mod 3, each wave its eight rows, in
  // kCvStages stages of at most one LDS access or a few VALU instructions, so they can sit between
  // MFMAs. Lane (row r = 8w + (l & 7), group gi = l >> 3) converts the group's 64 e4m3 values with
  // its ue8m0 scale: stage 0 reads the scale dword, 1-4 the four 16-byte source chunks, 5 forms the
  // scale, then each of the eight 16-byte writes takes three stages (two conversions of four
  // values, the write). For 512-wide rows group 7 is the RoPE tail, which those lanes copy to latent
  // columns 448-511 (a chunk read in the write's first stage). Each 16-lane quarter of a write meets
  // two-way bank conflicts (two groups 128 bytes apart); writing odd groups' upper halves first
  // would avoid them but its lane-dependent selects cost more than the conflicts.
  static constexpr int NG = kNope / 64;  // groups of e4m3 values per row
  static constexpr int kCvStages = 6 + 3 * 8;
  struct Cv {
    uint32_t sw;  // the row's scale dword holding the group's byte
    float sc;     // the group's scale
    u32x4 w[4];   // the group's e4m3 bytes
    bf16x8 x;     // the write in progress
    u32x4 rp;     // 512-wide rows, group 7: the RoPE chunk of the write in progress
    uint32_t src; // ring entry + the lane's first source chunk (chunk i: ^ 16 i; i only flips the
                  // two low bits of the swizzled chunk index)
    uint32_t dst; // bf16 slot + the lane's row and group
  };
  __device__ __forceinline__ void cv_stage(int st, Cv& c, int x, const Lane& L) const {
    const int ln = L.ln, r = 8 * wave + (ln & 7), gi = ln >> 3;
    const uint32_t re = ring_off(x);
    if (st == 0) {
      c.sw = *reinterpret_cast<const LDS_AS uint32_t*>(sm + re + kRingSc + 8 * r + (gi & 4));
      c.src = re + 512u * (uint32_t)r + 16u * (uint32_t)((4 * gi) ^ swz_ring(r));
      c.dst = slot_off(x) + (uint32_t)r * kRowStrideA + 128u * (uint32_t)gi;
    } else if (st <= 4) {
      const int i = st - 1;
      c.w[i] = *reinterpret_cast<const LDS_AS u32x4*>(sm + (c.src ^ (16u * (uint32_t)i)));
    } else if (st == 5) {
      c.sc = ue8m0_f32((c.sw >> (8 * (gi & 3))) & 0xFFu);
    } else {
      const int j = (st - 6) / 3, sub = (st - 6) % 3, i = j >> 1;
      const bool hi = (j & 1) != 0;  // this write: the upper 16 bytes of pair i
      if (sub == 0) {
        if constexpr (!HAS_B) {
          if (gi >= NG)
            c.rp = *reinterpret_cast<const LDS_AS u32x4*>(sm + re + kRingRope + 128u * (uint32_t)r + 16 * (2 * i + (hi ? 1 : 0)));
        }
        const uint32_t w0 = hi ? c.w[i][2] : c.w[i][0];
        const auto a0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, c.sc, false);
        const auto a1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, c.sc, true);
        c.x[0] = a0[0];
        c.x[1] = a0[1];
        c.x[2] = a1[0];
        c.x[3] = a1[1];
      } else if (sub == 1) {
        const uint32_t w1 = hi ? c.w[i][3] : c.w[i][1];
        const auto a2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, c.sc, false);
        const auto a3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, c.sc, true);
        c.x[4] = a2[0];
        c.x[5] = a2[1];
        c.x[6] = a3[0];
        c.x[7] = a3[1];
      } else {
        u32x4 v = __builtin_bit_cast(u32x4, c.x);
        if constexpr (!HAS_B) v = (gi < NG) ? v : c.rp;
        *reinterpret_cast<LDS_AS u32x4*>(sm + c.dst + 32u * (uint32_t)i + (hi ? 16u : 0u)) = v;
      }
    }
  }
  // PV slot (0-63) of conversion stage st
  __device__ __forceinline__ static constexpr int cv_slot(int st) { return (st * 64) / kCvStages; }
  __device__ __forceinline__ void convert_all(int x, const Lane& L) const {
    Cv c;
#pragma unroll
    for (int st = 0; st < kCvStages; ++st) cv_stage(st, c, x, L);
  }
  // bundle k landed, bundle k + 1 possibly still in flight (fp8 rows: the wave's own transfers of
  // bundle k + 1, the input of its conversion, landed; those of bundle k + 2, all issued among the
  // QK^T MFMAs, possibly in flight)
  __device__ __forceinline__ void wait_landed() const {
    asm volatile("s_waitcnt vmcnt(%0)" :: "n"(kNb) : "memory");
  }

  // ===== compute ===============================================================================
  // Q^T of the wave's two 16-row tiles of group g (rows past R repeat the last row; their outputs
  // are dropped)
  __device__ __forceinline__ void load_q(bf16x8 (&qr)[2][KS], int g) const {
    const int ln = lane_id();
    const int nl = ln & 15, gl = ln >> 4;
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const int r = min(mt * 128 + 32 * wave + 16 * nt + nl, a.R - 1);
      const bf16x8* src = reinterpret_cast<const bf16x8*>(a.q + ((int64_t)g * a.R + r) * DQK + 8 * gl);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) qr[nt][ks] = src[4 * ks];
    }
  }

  // Masks of a step's scores (lane row c = 16 kt + 4 gl + e of the step): valid iff (index lists)
  // its mask bit is set, or (dense) its position j = j0 + 32 t + c is inside the group's rows and
  // the query row's causal / window range.
  __device__ __forceinline__ void apply_mask(f32x4 (&s)[2][2], Cur c, int x, const Lane& L) const {
    const int ln = L.ln;
    const int nl = ln & 15, gl = ln >> 4;
    const uint32_t vmask = sparse ? *reinterpret_cast<const LDS_AS uint32_t*>(sm + kMOff + 4 * (x & 7)) : ~0u;
    bool need;
    if (sparse) {
      need = vmask != ~0u;
    } else {
      need = kRows * (c.t + 1) > c.n;  // past the group's rows
      if (!need && (a.causal || a.window > 0)) {
        // a whole step inside every query row's causal / window range needs no mask
        const int p0 = c.j0 + kRows * c.t, base = c.L - a.Sq;
        const bool in_c = !a.causal || p0 + kRows - 1 <= base + tok_lo;
        const bool in_w = a.window <= 0 || p0 >= base + tok_hi - a.window + 1;
        need = !(in_c && in_w);
      }
    }
    if (!need) return;
    if (sparse) {
      const uint32_t vm = vmask >> (4 * gl);
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const bool ok = ((vm >> (16 * kt + e)) & 1u) != 0;
#pragma unroll
          for (int nt = 0; nt < 2; ++nt) s[kt][nt][e] = ok ? s[kt][nt][e] : kNegInf;
        }
    } else {
      const int kbase = kRows * c.t + 4 * gl;  // step offset of e = 0, kt = 0
      const int nrem = c.n - kbase;
      int hi[2], lo[2];
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        // the query's position pos = L - Sq + token (token = row / H), relative to the step offset;
        // rows past R take row R - 1's (their Q^T is row R - 1's too)
        const uint32_t row = (uint32_t)min(mt * 128 + 32 * wave + 16 * nt + nl, a.R - 1);
        const int rel = c.L - a.Sq + (int)(row / (uint32_t)a.H) - c.j0 - kbase;
        hi[nt] = min(a.causal ? rel : (1 << 30), nrem - 1);  // the group's rows end at nrem
        lo[nt] = a.window > 0 ? rel - a.window + 1 : -(1 << 30);
      }
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int cc = 16 * kt + e;
#pragma unroll
          for (int nt = 0; nt < 2; ++nt) {
            const bool ok = (cc <= hi[nt]) & (cc >= lo[nt]);
            s[kt][nt][e] = ok ? s[kt][nt][e] : kNegInf;
          }
        }
    }
  }

  // Softmax of the wave's rows (base 2, lazy reference maximum) in micro-stages of at most two VALU
  // instructions or one exponential, so the QK^T loop of the next step can run one between each pair
  // of MFMAs (one wave hides about two VALU instructions under an MFMA): 0-3 row maxima, 4-6 their
  // reductions over the four lane groups (both row tiles through one permlane sequence), 8-13 the
  // reference updates, 14-29 the exponentials and sums (one value each), 30 the row sums.
  static constexpr int kSoftStages = 31;
  // Maxima of scores as single instructions: fmaxf would first quiet each operand that the compiler
  // cannot prove canonical (MFMA results from inline assembly, permlane results), one instruction
  // each. The scores are never NaN (finite inputs, -inf where masked).
  __device__ __forceinline__ static float max3_raw(float a, float b, float c) {
    float r;
    asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
  }
  __device__ __forceinline__ static float max_raw(float a, float b) {
    float r;
    asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
    return r;
  }
  __device__ __forceinline__ void soft_stage(int st, Soft& f, const f32x4 (&s)[2][2]) const {
    if (st < 4) {
      const int nt = st >> 1;
      if ((st & 1) == 0) {
        f.part[nt] = max3_raw(s[0][nt][0], s[0][nt][1], s[0][nt][2]);
        f.mx[nt] = max3_raw(s[0][nt][3], s[1][nt][0], s[1][nt][1]);
      } else {
        f.part[nt] = max3_raw(s[1][nt][2], s[1][nt][3], f.part[nt]);
        f.mx[nt] = max_raw(f.mx[nt], f.part[nt]);
      }
    } else if (st == 4) {
      // lane groups (rows of 16 lanes) r0..r3 hold partial maxima a (tile 0) and b (tile 1): swapping
      // a's odd rows with b's even rows leaves max(a.r0, a.r1), max(b.r0, b.r1), max(a.r2, a.r3),
      // max(b.r2, b.r3) in rows 0-3
      const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(f.mx[0]), __float_as_uint(f.mx[1]), false, false);
      f.mx[0] = max_raw(__uint_as_float(p[0]), __uint_as_float(p[1]));
    } else if (st == 5) {  // rows 0 and 2: tile 0's maximum; rows 1 and 3: tile 1's
      const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(f.mx[0]), __float_as_uint(f.mx[0]), false, false);
      f.mx[0] = max_raw(__uint_as_float(p[0]), __uint_as_float(p[1]));
    } else if (st == 6) {  // the even rows' value to every row, and the odd rows'
      const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(f.mx[0]), __float_as_uint(f.mx[0]), false, false);
      f.mx[0] = __uint_as_float(p[0]);
      f.mx[1] = __uint_as_float(p[1]);
    } else if (st >= 8 && st < 14) {
      const int nt = (st - 8) / 3, sub = (st - 8) % 3;
      if (sub == 0) {
        f.mnew[nt] = f.mx[nt] * a.scale_log2;  // -inf stays -inf (scale > 0)
        f.up[nt] = f.mnew[nt] > f.m_ref[nt] + kTau;
        if constexpr (MAXL) f.m_top[nt] = max_raw(f.m_top[nt], f.mnew[nt]);
      } else if (sub == 1) {
        f.alpha[nt] = f.up[nt] ? __builtin_amdgcn_exp2f(f.m_ref[nt] - f.mnew[nt]) : 1.f;  // m_ref = -inf -> 0
      } else {
        f.m_ref[nt] = f.up[nt] ? f.mnew[nt] : f.m_ref[nt];
        f.l_acc[nt] *= f.alpha[nt];
        f.mu[nt] = (f.m_ref[nt] == kNegInf) ? 0.f : f.m_ref[nt];
      }
    } else if (st >= 14 && st < 30) {
      const int v = st - 14, nt = v & 1, kt = (v >> 1) >> 2, e = (v >> 1) & 3;
      const float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kt][nt][e], a.scale_log2, -f.mu[nt]));
      f.lsum[nt] = (v < 2) ? pv : f.lsum[nt] + pv;  // the first term starts the sum
      f.pf[nt][kt * 4 + e] = (__bf16)pv;
    } else if (st == 30) {
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) f.l_acc[nt] += f.lsum[nt];
    }
  }
  __device__ __forceinline__ void soft_reset(Soft& f) const {
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      f.m_ref[nt] = kNegInf;
      f.l_acc[nt] = 0.f;
      f.m_top[nt] = kNegInf;
    }
  }

  // Side work of MFMA slot sl of an iteration (0 .. 4 KS - 1: QK^T, then 64 PV slots): the
  // transfers of the bundle being sent, one every kDmaGap slots, so the CU's LDS-DMA unit (about one
  // 1 KB transfer per 46 cycles) sees an even stream instead of bursts. fp8 rows send all of a
  // bundle among the QK^T MFMAs (the PV slots carry the conversion).
  static constexpr int kSlots = 4 * KS + 64;
  static constexpr int kDmaGap = (FP8 ? 4 * KS : kSlots) / kNb;  // fp8 rows: all among QK^T
  __device__ __forceinline__ int dma_part(int i) const { return (i < 8 || HAS_B) ? i : i + 1; }
  template <bool SEND>
  __device__ __forceinline__ void side_dma(int sl, int y, Cur cp, Cur cx, uint64_t& next, const DAddr& d,
                                           const Lane& L) const {
    if constexpr (SEND) {
      if (sl % kDmaGap == 1 && sl / kDmaGap < kNb) send_part(dma_part(sl / kDmaGap), y, cp, cx, next, d, L);
    }
  }

  // S^T = K Q^T of step x (slot x mod NS; fp8 rows: the RoPE part from ring entry x mod 3), with
  // the softmax micro-stages of the previous step (SOFT) and the first transfers of bundle y (SEND)
  // between the MFMAs.
  template <bool SOFT, bool SEND>
  __device__ __forceinline__ void qk(f32x4 (&sacc)[2][2], const bf16x8 (&qr)[2][KS], int x, Soft& f,
                                    const f32x4 (&sold)[2][2], int y, Cur cp, Cur cx, const DAddr& d,
                                    uint64_t& next, const Lane& L) const {
    const uint32_t sa = slot_off(x);
    const uint32_t sb = FP8 ? ring_off(x) + kRingRope : sa + kSlotA;
    const uint32_t kaddr = sa + L.kq();
    auto k_op = [&](int kt, int ks) -> bf16x8 {
      if (ks < 16) return lds_read_b128(sm, kaddr + 16 * kt * kRowStrideA + 64 * ks);
      // row 16 kt + nl, chunk (4 (ks - 16) + gl) ^ swz_b(row) (swz_b is the same for both kt)
      return lds_read_b128(sm, sb + (L.kr ^ (64u * (uint32_t)(ks - 16))) + 2048 * kt);
    };
    constexpr int D = 3;  // operand steps in flight
    bf16x8 ka[D][2];
#pragma unroll
    for (int i = 0; i < D - 1; ++i)
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) ka[i][kt] = k_op(kt, i);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int kt = m >> 1, nt = m & 1, sl = 4 * ks + m;
        if (ks + D - 1 < KS && nt == 0) ka[(ks + D - 1) % D][kt] = k_op(kt, ks + D - 1);
        if (ks == 0) mfma_s0(sacc[kt][nt], ka[ks % D][kt], qr[nt][ks]);
        else if (ks < KS - 1) mfma_s(sacc[kt][nt], ka[ks % D][kt], qr[nt][ks]);
        if constexpr (SOFT) {  // stages spread evenly over the 4 KS slots
#pragma unroll
          for (int st = 0; st < kSoftStages; ++st)
            if ((st * 4 * KS) / kSoftStages == sl) soft_stage(st, f, sold);
        }
        side_dma<SEND>(sl, y, cp, cx, next, d, L);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    constexpr int kl = (KS - 1) % D;
    mfma_s_last4(sacc[0][0], sacc[0][1], sacc[1][0], sacc[1][1], ka[kl][0], ka[kl][1], qr[0][KS - 1],
                 qr[1][KS - 1]);
  }

  // O^T (+)= V^T P^T of step x over all 512 output columns (FIRST: zero accumulator), with the rest
  // of bundle y's transfers between the MFMAs (SEND), or with fp8 rows the conversion of bundle
  // x + 2 (CV; WAIT: its transfers may still be in flight).
  template <bool FIRST, bool PREP, bool SEND, bool CV>
  __device__ __forceinline__ void pv(f32x4 (&o)[32][2], const bf16x8 (&pf)[2], int x, Cur c, int y, Cur cp,
                                    Cur cx, const DAddr& d, uint64_t& next, const Lane& L, bool wait) const {
    const uint32_t sa = slot_off(x);
    Cv cv;
    if constexpr (CV) {
      if (wait) wait_landed();
    }
    const uint32_t vbase = sa + L.vq();
    auto v_op = [&](int ct) -> bf16x8 {
      const uint32_t ad = vbase + 32 * ct;
      const bf16x4 v0 = lds_read_tr(sm, ad);
      const bf16x4 v1 = lds_read_tr(sm, ad + 16 * kRowStrideA);
      return __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
    };
    constexpr int VD = 4;
    bf16x8 va[VD];
#pragma unroll
    for (int i = 0; i < VD - 1; ++i) va[i] = v_op(i);
#pragma unroll
    for (int ct = 0; ct < 32; ++ct) {
      if (ct + VD - 1 < 32) va[(ct + VD - 1) % VD] = v_op(ct + VD - 1);
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const int sl = 4 * KS + 2 * ct + nt;
        if (FIRST) mfma_o0(o[ct][nt], va[ct % VD], pf[nt]);
        else mfma_o(o[ct][nt], va[ct % VD], pf[nt]);
        side_dma<SEND>(sl, y, cp, cx, next, d, L);
        if constexpr (CV) {
#pragma unroll
          for (int st = 0; st < kCvStages; ++st)
            if (cv_slot(st) == 2 * ct + nt) cv_stage(st, cv, x + 2, L);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }

  // rescale O^T where a row's reference maximum moved (rare once a split is under way)
  __device__ __forceinline__ void rescale(f32x4 (&o)[32][2], const Soft& f) const {
    if (!__any(f.up[0] | f.up[1])) return;
    mfma_drain_acc(o);
#pragma unroll
    for (int ct = 0; ct < 32; ++ct) {
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) o[ct][nt] *= f.alpha[nt];
      asm volatile("" : "+a"(o[ct][0]), "+a"(o[ct][1]));
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // One pipeline iteration k: QK^T of step k (cursor cq), softmax and PV of step k - 1 (cursor cs),
  // bundle k + 2 sent (its page and index steps: cp, cx), bundle k + 3 prepared (cursor cb; PREP);
  // EPI: step k - 1 ends its split, whose rows are then normalised and stored (`pin` runs before
  // the stores). A split boundary splits iteration k in two: its PV part (EPI, no PREP) ends the old
  // split, its QK part (no PV) starts the new one once that split's Q^T is loaded. WAIT: bundle k
  // may still be in flight (the first two steps of a split find their bundles landed: the
  // prologue, or the pin of the previous split's epilogue, waited for every load so far).
  struct NoPin {
    __device__ __forceinline__ void operator()() const {}
  };
  template <bool HAS_QK, bool HAS_PV, bool EPI, bool PREP, class Pin = NoPin>
  __device__ __forceinline__ void iteration(int k, bf16x8 (&qr)[2][KS], f32x4 (&o)[32][2], f32x4 (&sold)[2][2],
                                            f32x4 (&snew)[2][2],
                                            Soft& f, Cur& cq, Cur& cs, Cur& cb, Cur& cp, Cur& cx, DRows& dn,
                                            int cbase, bool wait, const Lane& L0, const Pin& pin = Pin()) {
    if constexpr (HAS_QK && !FP8) {
      if (wait) wait_landed();
    }
    // rows of step k visible (fp8 rows: converted in the previous iteration); every wave is done with
    // steps k - 2 (PV) and k - 1 (QK)
    lds_barrier();
    // The lane index is read again from the hardware (not held across the step); with fp8 rows, whose
    // conversion needs more registers, the other lane constants are worked out again as well.
    Lane L = FP8 ? make_lane() : L0;
    if constexpr (!FP8) {
      L.ln = lane_id();
      L.v16 = 16u * (uint32_t)L.ln;
    }
    DAddr da;
    if constexpr (HAS_QK && !SPARSE) da = dense_addr(dn);  // bundle k + 2 (entries loaded a step ago)
    if constexpr (HAS_PV) {
      if (cs.t == cs.q0) soft_reset(f);  // the softmax starts a new split
      apply_mask(sold, cs, k - 1, L);
    }
    const int ysend = cb.y - 1;  // bundle k + 2
    uint64_t next = 0;
    if constexpr (HAS_QK && SPARSE) next = rb_read(0);
    if constexpr (HAS_QK) {
      qk<HAS_PV, true>(snew, qr, k, f, sold, ysend, cp, cx, da, next, L);
    } else {
#pragma unroll
      for (int st = 0; st < kSoftStages; ++st) soft_stage(st, f, sold);
    }
    if constexpr (HAS_PV) {
      const bool first = cs.t == cs.q0;
      if (!first) rescale(o, f);
      asm volatile("s_nop 4" ::: "memory");  // P^T written by VALU, O^T rescaled: wait states
      // fp8 rows: bundle k + 1 converted among the MFMAs (its transfers issued an iteration ago)
      constexpr bool CV = FP8 && HAS_QK;
      if (first) pv<true, PREP, HAS_QK, CV>(o, f.pf, k - 1, cb, ysend, cp, cx, da, next, L, true);
      else pv<false, PREP, HAS_QK, CV>(o, f.pf, k - 1, cb, ysend, cp, cx, da, next, L, true);
      // index lists: the next bundle's addresses, once this bundle's transfers have read the table
      if constexpr (PREP && SPARSE) prepare(cb, L);
      if constexpr (EPI) {  // the split's last step: normalise and store its rows
        lds_barrier();  // every wave is done reading slot k - 1: it stages the epilogue
        epilogue(cbase + cs.ci, cs.g, desc(cs.ci, D_NSPLIT), slot_off(k - 1), o, f, L, pin);
      }
    } else {
      // no PV: the transfers placed among the PV MFMAs go out here
#pragma unroll
      for (int sl = 4 * KS; sl < kSlots; ++sl) side_dma<HAS_QK>(sl, ysend, cp, cx, next, da, L);
      if constexpr (PREP && SPARSE) prepare(cb, L);
      // fp8 rows: bundle k + 1, landed (the first step of a split: the prologue or the previous
      // split's epilogue waited for every load)
      if constexpr (FP8 && HAS_QK) convert_all(k + 1, L);
    }
    if constexpr (PREP) {
      if constexpr (!SPARSE) dn = dense_rows(cb);
      cb = cur_next(cb);
      if constexpr (SPARSE) {
        cp = cur_next(cp);
        cx = cur_next(cx);
      }
    }
    if constexpr (HAS_QK) {  // the caller swaps the roles of sold and snew for the next step
      cs = cq;
      cq = cur_next(cq);
    }
  }

  __device__ void run_chunk(int cb0) {
    const Cur c0 = cur_begin();
    Cur cb = c0, cp = c0, cx = c0;  // next bundle, block-table and index steps
    // ---- prologue: Q^T and sink logits of the first split, index and block-table entries,
    // bundles 0-1. Dense rows: Q^T, the sink logits and the bundles' rows are all in flight at
    // once (their one wait follows the transfers). -----------------------------------------------
    bf16x8 qr[2][KS];
    load_q(qr, c0.g);
    const Lane L0 = make_lane();
    Soft f;
    soft_reset(f);
    load_sink(f.sink, desc(c0.ci, D_NSPLIT), L0);
    if (sparse) {
#pragma unroll 1
      for (int i = 0; i < 6; ++i) {
        dma_dword(idx_src(cx), ix_slot(cx.y));
        cx = cur_next(cx);
      }
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll 1
      for (int i = 0; i < 3; ++i) {
        dma_dword(page_src(cp), pg_slot(cp.y));
        cp = cur_next(cp);
      }
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // entries in LDS before prepare reads them
    }
    DRows dn;
#pragma unroll 1
    for (int i = 0; i < 2; ++i) {
      DAddr d0;
      if constexpr (SPARSE) prepare(cb, L0);
      else d0 = dense_addr(dense_rows(cb));
      send_all(cb.y, cp, cx, d0, L0);
      cb = cur_next(cb);
      if constexpr (SPARSE) {
        cp = cur_next(cp);
        cx = cur_next(cx);
      }
    }
    if constexpr (SPARSE) prepare(cb, L0);  // bundle 2
    else dn = dense_rows(cb);
    cb = cur_next(cb);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) asm volatile("" : "+v"(qr[nt][ks]));  // Q^T has landed
    asm volatile("" : "+v"(f.sink[0]), "+v"(f.sink[1]));
    if constexpr (FP8) convert_all(0, L0);  // published by the first iteration's barrier

    f32x4 o[32][2];  // O^T: [output column tile][row tile], in accumulation registers
    f32x4 sa_[2][2], sb_[2][2];  // scores of a step, the two arrays taking turns as the new and old ones
    Cur cq = c0, cs = c0;
    // One pipelined loop per split. A split's Q^T is loaded between loops, so no loop holds a load
    // whose wait the compiler would place among the MFMAs (such a wait would also hold for the row
    // transfers in flight).
    int k = 0;
#pragma unroll 1
    for (int ci = 0; ci < nc; ++ci) {
      const int k0 = k, kend = k + (cq.qend - cq.q0);
      iteration<true, false, false, true>(k, qr, o, sb_, sa_, f, cq, cs, cb, cp, cx, dn, cb0, false, L0);
      // two steps per trip, so that the score arrays swap roles without copies
#pragma unroll 1
      for (++k; k + 1 < kend; k += 2) {
        iteration<true, true, false, true>(k, qr, o, sa_, sb_, f, cq, cs, cb, cp, cx, dn, cb0, k > k0 + 1, L0);
        iteration<true, true, false, true>(k + 1, qr, o, sb_, sa_, f, cq, cs, cb, cp, cx, dn, cb0, true, L0);
      }
      if (k < kend) {
        iteration<true, true, false, true>(k, qr, o, sa_, sb_, f, cq, cs, cb, cp, cx, dn, cb0, k > k0 + 1, L0);
        ++k;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int nt = 0; nt < 2; ++nt) sa_[kt][nt] = sb_[kt][nt];
      }
      // Q^T of the next split (cq: its first step) is requested before this split's last PV and
      // epilogue, which no longer need the registers, so it lands while they run. The epilogue waits
      // for it (and so for every load issued so far) before its stores, and the next split's sink
      // logits are requested after them, waited for only in its own epilogue: the stores drain
      // while the next split's first two steps run, which wait for no load. (After a chunk's last
      // split the epilogue's wait finds only zero-row bundles in flight.)
      if (ci + 1 < nc) load_q(qr, cq.g);
      auto pin = [&]() {
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) asm volatile("" : "+v"(qr[nt][ks]));
      };
      iteration<false, true, true, false>(k, qr, o, sa_, sb_, f, cq, cs, cb, cp, cx, dn, cb0, false, L0, pin);
      if (ci + 1 < nc) load_sink(f.sink, desc(cq.ci, D_NSPLIT), L0);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the epilogue's stores, zero-row bundles past the end
  }

  // Normalise the wave's 32 rows, stage them through slot LDS `stage` (16 rows x 256 columns at a
  // time) and store them as whole 128-byte lines, with their LSE; a group of one split gets its
  // final outputs (sink folded in), others partials. `pin` runs before the first store: it waits
  // for the loads the next split needs, so that no later wait has to cover the stores.
  //
  // Every lane stores, whatever R: a row past R holds the same values as row R - 1 (same Q row,
  // masks and sink; see load_q and apply_mask) and is stored there again, and the four lanes of a
  // row store its LSE alike. Each epilogue thus issues the same stores, none of them behind a
  // branch.
  template <class Pin>
  __device__ __forceinline__ void epilogue(int split, int g, int nsplit, uint32_t stage, f32x4 (&o)[32][2],
                                           const Soft& f, const Lane& L, const Pin& pin) const {
    mfma_drain_acc(o);
    const bool final_out = (nsplit == 1);
    const uint32_t wst = stage + wave * 16 * kStageRow;
    const int nl = L.ln & 15, gl = L.ln >> 4;
    float lse_nat[2], scale[2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) row_norm(f.sink[nt], f.m_ref[nt], rows_sum(f.l_acc[nt]), &lse_nat[nt], &scale[nt]);
    pin();
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const int r = min(mt * 128 + 32 * wave + 16 * nt + nl, a.R - 1);
      st_global_b32(final_out ? a.lse + lse_index(g, r) : a.part_lse + (int64_t)split * a.R + r, lse_nat[nt]);
      if constexpr (MAXL) {  // natural-log units of the scaled scores
        const float ml = f.m_top[nt] * 0.69314718055994530942f;
        st_global_b32(final_out ? a.max_logits + lse_index(g, r) : a.part_max + (int64_t)split * a.R + r, ml);
      }
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        // lane (nl, gl): columns 16 ct + 4 gl .. + 3 of row nl, ct in [16h, 16h + 16)
#pragma unroll
        for (int c = 0; c < 16; ++c) {
          const f32x4 v = acc_read(o[16 * h + c][nt]) * scale[nt];
          const u32x2 w = {(uint32_t)f2bf(v[0]) | ((uint32_t)f2bf(v[1]) << 16),
                           (uint32_t)f2bf(v[2]) | ((uint32_t)f2bf(v[3]) << 16)};
          *reinterpret_cast<LDS_AS u32x2*>(sm + wst + nl * kStageRow + 32 * c + 8 * gl) = w;
          __builtin_amdgcn_sched_barrier(0);
        }
        // lane l: 16 bytes at column 8 (l & 31) of staged row 2 i + (l >> 5)
        const int ln = L.ln;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int row = 2 * i + (ln >> 5);
          const u32x4 v = *reinterpret_cast<const LDS_AS u32x4*>(sm + wst + row * kStageRow + 16 * (ln & 31));
          const int rr = min(mt * 128 + 32 * wave + 16 * nt + row, a.R - 1);
          uint16_t* dst = final_out ? a.out + ((int64_t)g * a.R + rr) * kDv : a.part_o + ((int64_t)split * a.R + rr) * kDv;
          st_global_b128(dst + 256 * h + 8 * (ln & 31), v);
        }
      }
    }
  }

  // LSE (natural log) and output scale of a row; the sink logit sk (-inf: none) is folded in.
  __device__ __forceinline__ void row_norm(float sk, float m2, float l, float* lse_nat, float* scale) const {
    const float kLn2 = 0.69314718055994530942f;
    if (l > 0.f) {
      float lse = (m2 + __log2f(l)) * kLn2;
      float sc = 1.f / l;
      if (sk != kNegInf) {
        const float mx = fmaxf(lse, sk);
        const float lse2 = mx + __logf(__expf(lse - mx) + __expf(sk - mx));
        sc *= __expf(lse - lse2);
        lse = lse2;
      }
      *lse_nat = lse;
      *scale = sc;
    } else {
      *scale = 0.f;
      *lse_nat = sk;
    }
  }
  // Sink logits of the wave's two row tiles for a split's outputs (-inf: no sink, or partials that
  // the combine finishes). No wait here: the compiler waits for them where they are used (the
  // prologue's wait, or the epilogue before its stores).
  __device__ __forceinline__ void load_sink(float (&sk)[2], int nsplit, const Lane& L) const {
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const int r = min(mt * 128 + 32 * wave + 16 * nt + (L.ln & 15), a.R - 1);
      sk[nt] = (nsplit == 1 && a.sink != nullptr) ? a.sink[sparse ? r : r % a.H] : kNegInf;
    }
  }
  __device__ __forceinline__ int64_t lse_index(int g, int r) const {
    int bb, t, h;
    if (sparse) {
      bb = g / a.Sq;
      t = g % a.Sq;
      h = r;
    } else {
      bb = g;
      t = r / a.H;
      h = r % a.H;
    }
    return ((int64_t)bb * a.H + h) * a.Sq + t;
  }

  __device__ void run_unit(int s0, int s1) {
#pragma unroll 1
    for (int cb = s0; cb < s1; cb += kChunk) {
      nc = min(kChunk, s1 - cb);
      lds_barrier();  // every wave is done with the previous chunk's table and slots
      build_table(cb);
      lds_barrier();
      T = 0;
#pragma unroll 1
      for (int ci = 0; ci < nc; ++ci) T += desc(ci, D_QEND) - desc(ci, D_Q0);
      run_chunk(cb);
    }
  }
};

// Workgroup b -> (unit, row tile) for the 128-row kernel: workgroups are dealt to the 8 XCDs
// round-robin; XCD x takes units [x * per, (x + 1) * per), all row tiles of a unit together, so the
// splits of one request (consecutive units) share one L2 for their Q rows and block-table entries.
__device__ __forceinline__ void unit_tile_blocked(int bid, int m_tiles, int per, int* unit, int* mt) {
  const int x = bid & 7, q = bid >> 3;
  *mt = q % m_tiles;
  *unit = x * per + q / m_tiles;
}

template <int DQK, bool MAXL, bool SPARSE, bool FP8>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void decode_tile128_kernel(DecodeArgs a, int per) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[Tile128<DQK, MAXL, SPARSE, FP8>::LDS];
  int unit, mt;
  unit_tile_blocked(blockIdx.x, a.m_tiles, per, &unit, &mt);
  int s0, s1;
  if (!unit_splits<!MAXL>(a, unit, &s0, &s1)) return;
  Tile128<DQK, MAXL, SPARSE, FP8> d(a, (lds_ptr)lds, mt);
  d.run_unit(s0, s1);
}

// Workgroup b -> (unit, row tile): all row tiles of a unit land on the same XCD (workgroups are
// dealt to the 8 XCDs round-robin), so the second reader of a KV block finds it in that L2.
__device__ __forceinline__ void unit_tile(int bid, int m_tiles, int* unit, int* mt) {
  const int x = bid & 7, q = bid >> 3;
  *mt = q % m_tiles;
  *unit = (q / m_tiles) * 8 + x;
}

template <int DQK, bool FP8>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void decode_spec64_kernel(DecodeArgs a) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[Spec64<DQK, FP8>::LDS];
  const lds_ptr base = (lds_ptr)lds;
  int unit, mt;
  unit_tile(blockIdx.x, a.m_tiles, &unit, &mt);
  int s0, s1;
  if (!unit_splits(a, unit, &s0, &s1)) return;
  Spec64<DQK, FP8> d(a, base);
  if (d.wave < 4) {
    for (int s = s0; s < s1; ++s) {
      d.load_split(s);
      d.score_split(mt);
    }
  } else {
    for (int s = s0; s < s1; ++s) {
      d.load_split(s);
      d.value_split(s, mt);
    }
  }
}

template <class C>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void decode_kernel(DecodeArgs a) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[C::LDS];
  const lds_ptr base = (lds_ptr)lds;
  const int m_tiles = a.m_tiles;
  const int unit = blockIdx.x / m_tiles;
  const int mt = blockIdx.x % m_tiles;
  int s0, s1;
  if (!unit_splits<false>(a, unit, &s0, &s1)) return;
  Decoder<C> d(a, base);
  for (int s = s0; s < s1; ++s) d.run_split(s, mt);
}

// The kernel's row tile may be smaller than the plan's: the grid then holds one workgroup per
// (unit, kernel row tile), all of a unit's workgroups walking the same splits.
template <class C>
hipError_t launch_cfg(DecodeArgs a, hipStream_t s) {
  a.m_tiles = (a.R + C::M_TILE - 1) / C::M_TILE;
  const int64_t grid = (int64_t)a.U * a.m_tiles;
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL(decode_kernel<C>, dim3((unsigned)grid), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

template <int DQK, bool FP8>
hipError_t launch_spec64(DecodeArgs a, hipStream_t s) {
  a.m_tiles = (a.R + 63) / 64;
  const int64_t grid = (int64_t)((a.U + 7) / 8) * 8 * a.m_tiles;
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL((decode_spec64_kernel<DQK, FP8>), dim3((unsigned)grid), dim3(512), 0, s, a);
  return hipGetLastError();
}

template <int DQK, bool SPARSE>
hipError_t launch_tile128_t(const DecodeArgs& a, int per, int64_t grid, hipStream_t s) {
  if (a.max_logits != nullptr)
    hipLaunchKernelGGL((decode_tile128_kernel<DQK, true, SPARSE, false>), dim3((unsigned)grid), dim3(256), 0, s, a, per);
  else
    hipLaunchKernelGGL((decode_tile128_kernel<DQK, false, SPARSE, false>), dim3((unsigned)grid), dim3(256), 0, s, a, per);
  return hipGetLastError();
}
template <int DQK>
hipError_t launch_tile128(DecodeArgs a, hipStream_t s, bool fp8) {
  a.m_tiles = (a.R + 127) / 128;
  const int per = (a.U + 7) / 8;
  const int64_t grid = (int64_t)8 * per * a.m_tiles;
  if (grid <= 0) return hipSuccess;
  if (fp8) {
    hipLaunchKernelGGL((decode_tile128_kernel<DQK, false, false, true>), dim3((unsigned)grid), dim3(256), 0, s, a, per);
    return hipGetLastError();
  }
  return a.topk > 0 ? launch_tile128_t<DQK, true>(a, per, grid, s) : launch_tile128_t<DQK, false>(a, per, grid, s);
}

// 65+ stacked rows run on the 128-row tile unless the problem is known to give each unit under
// four blocks (index lists of a few blocks, short windows, few groups): such short splits run
// faster on 64-row tiles, whose per-split prologue (Q rows) and epilogue are half as long. Without
// a window or index lists the row counts are only known on the device, and the 128-row tile is
// taken.
inline bool prefer_tile128(const Shape& sh) {
  if (sh.R <= 64) return false;
  int64_t blocks_per_group = -1;
  if (sh.topk > 0) blocks_per_group = (sh.topk + kBlockRows - 1) / kBlockRows;
  else if (sh.window > 0) blocks_per_group = (int64_t)(sh.window + sh.Sq - 1 + kBlockRows - 1) / kBlockRows + 1;
  return blocks_per_group < 0 || (int64_t)sh.G * blocks_per_group >= 4 * (int64_t)sh.U;
}

template <int DQK>
hipError_t launch_dqk(const DecodeArgs& a, const Shape& sh, hipStream_t s) {
  const bool t128 = prefer_tile128(sh);
  if (sh.fmt == 0 && t128) return launch_tile128<DQK>(a, s, false);  // bf16 rows
  // fp8 rows, dense: converted once per step into bf16 slots
  if (sh.fmt != 0 && t128 && a.topk == 0 && a.max_logits == nullptr) return launch_tile128<DQK>(a, s, true);
  if (sh.fmt != 0) return launch_spec64<DQK, true>(a, s);  // other fp8 rows: 64-row tiles
  if (a.max_logits == nullptr) {  // the per-row maximum is produced by the 64-row kernel only
    if (sh.R <= 16) return launch_cfg<Cfg<16, 4, DQK>>(a, s);
    if (sh.R <= 32) return launch_cfg<Cfg<16, 2, DQK>>(a, s);
  }
  return launch_spec64<DQK, false>(a, s);
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, const Shape& sh, hipStream_t s) {
  return sh.d_qk == 576 ? launch_dqk<576>(a, sh, s) : launch_dqk<512>(a, sh, s);
}

}  // namespace mla
