// C ABI of the MLA decode library (include/mla.h): argument checks, workspace sizing, plan layout
// and kernel dispatch. Every check runs on the host before anything is enqueued.
#include "../../include/mla.h"
#include "mla_internal.h"
#include "layer_internal.h"

#include <math.h>

#include <atomic>
#include <mutex>

// Hash of the sources the library was built from (set by the build; see mla_build_id).
#ifndef MLA_BUILD_ID
#define MLA_BUILD_ID "unknown"
#endif

using mla::PlanLayout;
using mla::Shape;

namespace {

bool is_pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int query_cus(int32_t* out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MLA_ERR_DEVICE;
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return MLA_ERR_DEVICE;
  *out = cus;
  return MLA_OK;
}

// Validate a problem and derive its shape. num_cus <= 0 queries the device.
int derive(const mla_problem* p, int32_t num_cus, Shape* sh) {
  if (p == nullptr || sh == nullptr) return MLA_ERR_NULL;
  if (p->batch < 1 || p->q_len < 1 || p->num_heads < 1) return MLA_ERR_SHAPE;
  if (p->d_v != 512 || p->d_rope != 64) return MLA_ERR_SHAPE;
  if (p->d_qk != 576 && p->d_qk != 512) return MLA_ERR_SHAPE;
  if (p->kv_format != MLA_KV_BF16 && p->kv_format != MLA_KV_FP8) return MLA_ERR_FORMAT;
  if (!is_pow2(p->page_size) || p->page_size > 4096) return MLA_ERR_PAGE;
  if (p->topk < 0 || p->window < 0 || (p->causal != 0 && p->causal != 1)) return MLA_ERR_MODE;
  if (p->topk > 0 && (p->causal != 0 || p->window != 0)) return MLA_ERR_MODE;
  if (p->max_pages_per_seq < 1 || p->num_pages < 1 || p->num_pages > INT32_MAX) return MLA_ERR_PAGE;
  const int64_t d_nope = p->d_qk - p->d_rope;
  const int64_t row_bytes = (p->kv_format == MLA_KV_BF16) ? 2LL * p->d_qk : d_nope + 2LL * p->d_rope;
  const int64_t used = (int64_t)p->page_size * (row_bytes + (p->kv_format == MLA_KV_FP8 ? 8 : 0));
  if (p->page_stride_bytes < used || (p->page_stride_bytes & 15) != 0) return MLA_ERR_PAGE;

  const int64_t R = (p->topk > 0) ? (int64_t)p->num_heads : (int64_t)p->q_len * p->num_heads;
  const int64_t G = (p->topk > 0) ? (int64_t)p->batch * p->q_len : (int64_t)p->batch;
  if (R > 65536 || G > mla::kMaxGroups) return MLA_ERR_SHAPE;
  if (num_cus <= 0) {
    int rc = query_cus(&num_cus);
    if (rc != MLA_OK) return rc;
  }
  int m_tile = 0, fixed = 0;
  mla::tile_params((int)R, &m_tile, &fixed);
  sh->B = p->batch;
  sh->Sq = p->q_len;
  sh->H = p->num_heads;
  sh->R = (int)R;
  sh->G = (int)G;
  sh->m_tile = m_tile;
  sh->fixed = fixed;
  sh->m_tiles = (int)((R + m_tile - 1) / m_tile);
  sh->U = num_cus / sh->m_tiles;
  if (sh->U < 1) sh->U = 1;
  sh->d_qk = p->d_qk;
  sh->d_rope = p->d_rope;
  sh->fmt = p->kv_format;
  sh->page_size = p->page_size;
  int lg = 0;
  while ((1 << lg) < p->page_size) ++lg;
  sh->ps_log2 = lg;
  sh->max_pages = p->max_pages_per_seq;
  sh->topk = p->topk;
  sh->causal = p->causal;
  sh->window = p->window;
  sh->page_stride = p->page_stride_bytes;
  sh->num_pages = p->num_pages;
  sh->row_bytes = row_bytes;
  sh->s_max = (int64_t)sh->G + sh->U;
  return MLA_OK;
}

size_t partial_size(const Shape& sh) {
  // bf16 partial O rows, then fp32 partial LSEs
  return (size_t)sh.s_max * (size_t)sh.R * ((size_t)mla::kDv * sizeof(uint16_t) + sizeof(float));
}

int launch_rc(hipError_t e) { return e == hipSuccess ? MLA_OK : MLA_ERR_LAUNCH; }

std::atomic<bool> g_checked{false};  // checked mode (mla_check_enable)

}  // namespace

extern "C" {

int mla_device_num_cus(int32_t* num_cus) {
  if (num_cus == nullptr) return MLA_ERR_NULL;
  return query_cus(num_cus);
}

int mla_get_workspace_size(const mla_problem* p, int32_t num_cus, size_t* plan_bytes,
                           size_t* partial_bytes) {
  Shape sh;
  int rc = derive(p, num_cus, &sh);
  if (rc != MLA_OK) return rc;
  if (plan_bytes) *plan_bytes = (size_t)PlanLayout::make(sh.G, sh.U).bytes;
  if (partial_bytes) *partial_bytes = partial_size(sh);
  return MLA_OK;
}

int mla_decode_plan(const mla_problem* p, int32_t num_cus, const int32_t* seqlens,
                    const int32_t* topk_lens, void* plan, size_t plan_bytes, void* stream) {
  Shape sh;
  int rc = derive(p, num_cus, &sh);
  if (rc != MLA_OK) return rc;
  if (seqlens == nullptr || plan == nullptr) return MLA_ERR_NULL;
  if (!aligned16(plan)) return MLA_ERR_ALIGN;
  const PlanLayout lay = PlanLayout::make(sh.G, sh.U);
  if (plan_bytes < (size_t)lay.bytes) return MLA_ERR_WORKSPACE;
  mla::PlanArgs a;
  a.seqlens = seqlens;
  a.topk_lens = (sh.topk > 0) ? topk_lens : nullptr;
  a.plan = static_cast<int32_t*>(plan);
  a.lay = lay;
  a.B = sh.B;
  a.Sq = sh.Sq;
  a.R = sh.R;
  a.G = sh.G;
  a.U = sh.U;
  a.m_tiles = sh.m_tiles;
  a.m_tile = sh.m_tile;
  a.fixed = sh.fixed;
  a.topk = sh.topk;
  a.window = sh.window;
  return launch_rc(mla::launch_plan(a, static_cast<hipStream_t>(stream)));
}

}  // extern "C"

namespace {

// mla_decode with an optional per-row maximum (max_logits, with part_max holding S_max * R floats
// for the split rows).
int decode_impl(const mla_problem* p, int32_t num_cus, const void* q, const void* kv_cache,
                const int32_t* block_table, const int32_t* seqlens, float sm_scale,
                const int32_t* indices, const float* sink, const void* plan, void* partials,
                size_t partial_bytes, void* out, float* lse, float* max_logits, float* part_max,
                void* stream) {
  Shape sh;
  int rc = derive(p, num_cus, &sh);
  if (rc != MLA_OK) return rc;
  if (q == nullptr || kv_cache == nullptr || block_table == nullptr || seqlens == nullptr ||
      plan == nullptr || out == nullptr || lse == nullptr)
    return MLA_ERR_NULL;
  if (sh.topk > 0 && indices == nullptr) return MLA_ERR_NULL;
  if (!aligned16(q) || !aligned16(kv_cache) || !aligned16(plan) || !aligned16(out) ||
      (partials != nullptr && !aligned16(partials)))
    return MLA_ERR_ALIGN;
  if (!(sm_scale > 0.f) || !isfinite(sm_scale)) return MLA_ERR_SHAPE;
  const size_t need = partial_size(sh);
  if (partials == nullptr || partial_bytes < need) return MLA_ERR_WORKSPACE;
  const PlanLayout lay = PlanLayout::make(sh.G, sh.U);
  mla::DecodeArgs a;
  a.q = static_cast<const uint16_t*>(q);
  a.cache = static_cast<const uint8_t*>(kv_cache);
  a.block_table = block_table;
  a.seqlens = seqlens;
  a.indices = (sh.topk > 0) ? indices : nullptr;
  a.sink = sink;
  a.plan = static_cast<const int32_t*>(plan);
  a.zero_row = static_cast<const uint8_t*>(plan) + lay.zero_row_bytes_off;
  a.part_o = static_cast<uint16_t*>(partials);
  a.part_lse = reinterpret_cast<float*>(a.part_o + (size_t)sh.s_max * sh.R * mla::kDv);
  a.out = static_cast<uint16_t*>(out);
  a.lse = lse;
  a.max_logits = max_logits;
  a.part_max = part_max;
  a.page_stride = sh.page_stride;
  a.num_pages = sh.num_pages;
  a.row_bytes = sh.row_bytes;
  a.scale_off = (int64_t)sh.page_size * sh.row_bytes;
  a.grp_ptr_off = lay.grp_ptr;
  a.unit_ptr_off = lay.unit_ptr;
  a.grp_rows_off = lay.grp_rows;
  a.splits_off = lay.splits;
  a.sdesc_off = lay.sdesc_bytes_off / 4;
  a.B = sh.B;
  a.Sq = sh.Sq;
  a.H = sh.H;
  a.R = sh.R;
  a.G = sh.G;
  a.U = sh.U;
  a.m_tiles = sh.m_tiles;
  a.ps_log2 = sh.ps_log2;
  a.max_pages = sh.max_pages;
  a.topk = sh.topk;
  a.causal = sh.causal;
  a.window = sh.window;
  a.scale_log2 = sm_scale * 1.4426950408889634f;
  if (g_checked.load(std::memory_order_relaxed)) {
    mla::CheckArgs c;
    c.plan = a.plan;
    c.block_table = block_table;
    c.seqlens = seqlens;
    c.indices = a.indices;
    c.num_pages = sh.num_pages;
    c.grp_rows_off = lay.grp_rows;
    c.B = sh.B;
    c.Sq = sh.Sq;
    c.R = sh.R;
    c.G = sh.G;
    c.U = sh.U;
    c.ps_log2 = sh.ps_log2;
    c.max_pages = sh.max_pages;
    c.topk = sh.topk;
    c.window = sh.window;
    rc = launch_rc(mla::launch_check(c, static_cast<hipStream_t>(stream)));
    if (rc != MLA_OK) return rc;
  }
  return launch_rc(mla::launch_decode(a, sh, static_cast<hipStream_t>(stream)));
}

int combine_impl(const mla_problem* p, int32_t num_cus, const void* plan, const void* partials,
                 size_t partial_bytes, const float* sink, void* out, float* lse,
                 const float* part_max, float* max_logits, void* stream) {
  Shape sh;
  int rc = derive(p, num_cus, &sh);
  if (rc != MLA_OK) return rc;
  if (plan == nullptr || out == nullptr || lse == nullptr) return MLA_ERR_NULL;
  if (!aligned16(plan) || !aligned16(out) || (partials != nullptr && !aligned16(partials)))
    return MLA_ERR_ALIGN;
  if (partials == nullptr || partial_bytes < partial_size(sh)) return MLA_ERR_WORKSPACE;
  const PlanLayout lay = PlanLayout::make(sh.G, sh.U);
  mla::CombineArgs a;
  a.plan = static_cast<const int32_t*>(plan);
  a.part_o = static_cast<const uint16_t*>(partials);
  a.part_lse = reinterpret_cast<const float*>(a.part_o + (size_t)sh.s_max * sh.R * mla::kDv);
  a.sink = sink;
  a.out = static_cast<uint16_t*>(out);
  a.lse = lse;
  a.part_max = part_max;
  a.max_logits = max_logits;
  a.grp_ptr_off = lay.grp_ptr;
  a.B = sh.B;
  a.Sq = sh.Sq;
  a.H = sh.H;
  a.R = sh.R;
  a.G = sh.G;
  a.U = sh.U;
  a.sparse = sh.topk > 0;
  return launch_rc(mla::launch_combine(a, static_cast<hipStream_t>(stream)));
}

size_t round256(size_t x) { return (x + 255) / 256 * 256; }

// The sparse prefill as one request over the flat buffer: its positions are kv's rows, pages of
// 4096 rows, page i at page i. Workspace: [s_kv, identity page table] | plan | partials | split
// maxima, each part 256-byte aligned.
struct SparseLayout {
  mla_problem p;
  Shape sh;
  int32_t pages;
  size_t plan_off, plan_bytes, part_off, part_bytes, max_off, bytes;
};

int sparse_layout(int32_t s_q, int32_t num_heads, int32_t d_qk, int32_t topk, int64_t s_kv,
                  int32_t num_cus, SparseLayout* L) {
  if (s_q < 1 || topk < 1 || s_kv < 1 || s_kv > INT32_MAX) return MLA_ERR_SHAPE;
  constexpr int32_t kPage = 4096;
  mla_problem& p = L->p;
  p.batch = 1;
  p.q_len = s_q;
  p.num_heads = num_heads;
  p.d_qk = d_qk;
  p.d_v = 512;
  p.d_rope = 64;
  p.kv_format = MLA_KV_BF16;
  p.page_size = kPage;
  p.page_stride_bytes = (int64_t)kPage * 2 * d_qk;
  p.num_pages = (s_kv + kPage - 1) / kPage;
  p.max_pages_per_seq = (int32_t)p.num_pages;
  p.topk = topk;
  p.causal = 0;
  p.window = 0;
  int rc = derive(&p, num_cus, &L->sh);
  if (rc != MLA_OK) return rc;
  L->pages = (int32_t)p.num_pages;
  L->plan_off = round256(sizeof(int32_t) * (1 + (size_t)L->pages));
  L->plan_bytes = (size_t)PlanLayout::make(L->sh.G, L->sh.U).bytes;
  L->part_off = round256(L->plan_off + L->plan_bytes);
  L->part_bytes = partial_size(L->sh);
  L->max_off = round256(L->part_off + L->part_bytes);
  L->bytes = L->max_off + (size_t)L->sh.s_max * L->sh.R * sizeof(float);
  return MLA_OK;
}

}  // namespace

extern "C" {

int mla_decode(const mla_problem* p, int32_t num_cus, const void* q, const void* kv_cache,
               const int32_t* block_table, const int32_t* seqlens, float sm_scale,
               const int32_t* indices, const float* sink, const void* plan, void* partials,
               size_t partial_bytes, void* out, float* lse, void* stream) {
  return decode_impl(p, num_cus, q, kv_cache, block_table, seqlens, sm_scale, indices, sink, plan,
                     partials, partial_bytes, out, lse, nullptr, nullptr, stream);
}

int mla_combine(const mla_problem* p, int32_t num_cus, const void* plan, const void* partials,
                size_t partial_bytes, const float* sink, void* out, float* lse, void* stream) {
  return combine_impl(p, num_cus, plan, partials, partial_bytes, sink, out, lse, nullptr, nullptr,
                      stream);
}

}  // extern "C"

namespace {

// Device scratch of mla_decode_noalloc: the plan, then the split partials, of the last call on each
// device. A file-scope device array exists once per GPU the library runs on and lives until the
// process ends. In host code `scratch` names a host-side stand-in, so its device address is taken
// once per device with hipGetSymbolAddress and only that address is used.
constexpr size_t kScratchBytes = size_t(64) << 20;
__device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices];

// Device address of the current device's scratch (resolved on the first call on that device).
int scratch_address(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MLA_ERR_DEVICE;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr)
      return MLA_ERR_DEVICE;
    g_scratch[dev] = ptr;
  }
  *out = g_scratch[dev];
  return MLA_OK;
}

}  // namespace

extern "C" {

int mla_decode_noalloc(const mla_problem* p, int32_t num_cus, const void* q, const void* kv_cache,
                       const int32_t* block_table, const int32_t* seqlens,
                       const int32_t* topk_lens, float sm_scale, const int32_t* indices,
                       const float* sink, void* out, float* lse, void* stream) {
  Shape sh;
  int rc = derive(p, num_cus, &sh);
  if (rc != MLA_OK) return rc;
  if (num_cus <= 0) {
    rc = query_cus(&num_cus);
    if (rc != MLA_OK) return rc;
  }
  const size_t plan_bytes = round256((size_t)PlanLayout::make(sh.G, sh.U).bytes);
  const size_t part_bytes = partial_size(sh);
  if (plan_bytes + part_bytes > kScratchBytes) return MLA_ERR_SCRATCH;
  // the same host checks as the calls it stands for, before anything is enqueued
  if (q == nullptr || kv_cache == nullptr || block_table == nullptr || seqlens == nullptr ||
      out == nullptr || lse == nullptr || (sh.topk > 0 && indices == nullptr))
    return MLA_ERR_NULL;
  if (!aligned16(q) || !aligned16(kv_cache) || !aligned16(out)) return MLA_ERR_ALIGN;
  if (!(sm_scale > 0.f) || !isfinite(sm_scale)) return MLA_ERR_SHAPE;
  void* base = nullptr;
  rc = scratch_address(&base);
  if (rc != MLA_OK) return rc;
  uint8_t* plan = static_cast<uint8_t*>(base);
  uint8_t* partials = plan + plan_bytes;
  rc = mla_decode_plan(p, num_cus, seqlens, topk_lens, plan, plan_bytes, stream);
  if (rc != MLA_OK) return rc;
  rc = decode_impl(p, num_cus, q, kv_cache, block_table, seqlens, sm_scale, indices, sink, plan,
                   partials, part_bytes, out, lse, nullptr, nullptr, stream);
  if (rc != MLA_OK) return rc;
  return combine_impl(p, num_cus, plan, partials, part_bytes, sink, out, lse, nullptr, nullptr,
                      stream);
}

int mla_sparse_prefill_workspace_size(int32_t s_q, int32_t num_heads, int32_t d_qk, int32_t topk,
                                      int64_t s_kv, int32_t num_cus, size_t* workspace_bytes) {
  SparseLayout L;
  int rc = sparse_layout(s_q, num_heads, d_qk, topk, s_kv, num_cus, &L);
  if (rc != MLA_OK) return rc;
  if (workspace_bytes) *workspace_bytes = L.bytes;
  return MLA_OK;
}

int mla_sparse_prefill(int32_t s_q, int32_t num_heads, int32_t d_qk, int32_t topk, int64_t s_kv,
                       int32_t num_cus, const void* q, const void* kv, const int32_t* indices,
                       float sm_scale, void* workspace, size_t workspace_bytes, void* out,
                       float* max_logits, float* lse, void* stream) {
  SparseLayout L;
  int rc = sparse_layout(s_q, num_heads, d_qk, topk, s_kv, num_cus, &L);
  if (rc != MLA_OK) return rc;
  if (q == nullptr || kv == nullptr || indices == nullptr || workspace == nullptr ||
      out == nullptr || max_logits == nullptr || lse == nullptr)
    return MLA_ERR_NULL;
  if (!aligned16(q) || !aligned16(kv) || !aligned16(workspace) || !aligned16(out))
    return MLA_ERR_ALIGN;
  if (!(sm_scale > 0.f) || !isfinite(sm_scale)) return MLA_ERR_SHAPE;
  if (workspace_bytes < L.bytes) return MLA_ERR_WORKSPACE;
  if (num_cus <= 0) {
    rc = query_cus(&num_cus);
    if (rc != MLA_OK) return rc;
  }
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  int32_t* meta = reinterpret_cast<int32_t*>(ws);
  void* plan = ws + L.plan_off;
  void* partials = ws + L.part_off;
  float* part_max = reinterpret_cast<float*>(ws + L.max_off);
  hipStream_t st = static_cast<hipStream_t>(stream);
  rc = launch_rc(mla::launch_sparse_meta(meta, (int32_t)s_kv, L.pages, st));
  if (rc != MLA_OK) return rc;
  rc = mla_decode_plan(&L.p, num_cus, meta, nullptr, plan, L.plan_bytes, stream);
  if (rc != MLA_OK) return rc;
  rc = decode_impl(&L.p, num_cus, q, kv, meta + 1, meta, sm_scale, indices, nullptr, plan,
                   partials, L.part_bytes, out, lse, max_logits, part_max, stream);
  if (rc != MLA_OK) return rc;
  return combine_impl(&L.p, num_cus, plan, partials, L.part_bytes, nullptr, out, lse, part_max,
                      max_logits, stream);
}

int mla_kv_write(const mla_problem* p, int64_t num_tokens, const void* kv_c, const void* k_pe,
                 const int64_t* slot_mapping, void* kv_cache, void* stream) {
  Shape sh;
  int rc = derive(p, 1, &sh);
  if (rc != MLA_OK) return rc;
  if (num_tokens < 0 || num_tokens > (int64_t)INT32_MAX) return MLA_ERR_SHAPE;
  if (num_tokens == 0) return MLA_OK;
  if (kv_c == nullptr || k_pe == nullptr || slot_mapping == nullptr || kv_cache == nullptr)
    return MLA_ERR_NULL;
  if (!aligned16(kv_c) || !aligned16(k_pe) || !aligned16(kv_cache) ||
      (reinterpret_cast<uintptr_t>(slot_mapping) & 7u) != 0)
    return MLA_ERR_ALIGN;
  mla::KvWriteArgs a;
  a.kv_c = static_cast<const uint16_t*>(kv_c);
  a.k_pe = static_cast<const uint16_t*>(k_pe);
  a.slots = slot_mapping;
  a.cache = static_cast<uint8_t*>(kv_cache);
  a.n = num_tokens;
  a.num_slots = sh.num_pages * (int64_t)sh.page_size;
  a.page_stride = sh.page_stride;
  a.scale_off = (int64_t)sh.page_size * sh.row_bytes;
  a.ps_log2 = sh.ps_log2;
  return launch_rc(mla::launch_kv_write(a, sh.fmt, sh.d_qk - sh.d_rope,
                                        static_cast<hipStream_t>(stream)));
}
int mla_q_absorb(int32_t tokens, int32_t num_heads, int32_t d_nope, int32_t d_latent,
                 int32_t d_rope, const void* q_nope, const void* q_pe, const void* w_uk, void* q_out,
                 void* stream) {
  if (tokens < 0 || num_heads < 1 || d_nope < 32 || d_nope % 32 != 0 || d_latent < 64 ||
      d_latent % 64 != 0 || d_rope < 0 || d_rope % 8 != 0 || num_heads > 65535)
    return MLA_ERR_SHAPE;
  if (tokens == 0) return MLA_OK;
  if (q_nope == nullptr || w_uk == nullptr || q_out == nullptr || (d_rope > 0 && q_pe == nullptr))
    return MLA_ERR_NULL;
  if (!aligned16(q_nope) || !aligned16(w_uk) || !aligned16(q_out) ||
      (d_rope > 0 && !aligned16(q_pe)))
    return MLA_ERR_ALIGN;
  mla::GemmArgs a;
  a.a = static_cast<const uint16_t*>(q_nope);
  a.a_t = (int64_t)num_heads * d_nope;
  a.a_h = d_nope;
  a.w = static_cast<const uint16_t*>(w_uk);
  a.c = static_cast<uint16_t*>(q_out);
  a.c_h = (int64_t)d_latent + d_rope;
  a.c_t = (int64_t)num_heads * a.c_h;
  a.pe = d_rope > 0 ? static_cast<const uint16_t*>(q_pe) : nullptr;
  a.pe_t = (int64_t)num_heads * d_rope;
  a.pe_h = d_rope;
  a.T = tokens;
  a.H = num_heads;
  a.N = d_latent;
  a.K = d_nope;
  a.R = d_rope;
  return launch_rc(mla::launch_absorb_gemm(a, static_cast<hipStream_t>(stream)));
}
int mla_v_up(int32_t tokens, int32_t num_heads, int32_t d_latent, int32_t d_v, const void* o,
             const void* w_uv, void* out, void* stream) {
  if (tokens < 0 || num_heads < 1 || d_latent < 32 || d_latent % 32 != 0 || d_v < 64 ||
      d_v % 64 != 0 || num_heads > 65535)
    return MLA_ERR_SHAPE;
  if (tokens == 0) return MLA_OK;
  if (o == nullptr || w_uv == nullptr || out == nullptr) return MLA_ERR_NULL;
  if (!aligned16(o) || !aligned16(w_uv) || !aligned16(out)) return MLA_ERR_ALIGN;
  mla::GemmArgs a;
  a.a = static_cast<const uint16_t*>(o);
  a.a_t = (int64_t)num_heads * d_latent;
  a.a_h = d_latent;
  a.w = static_cast<const uint16_t*>(w_uv);
  a.c = static_cast<uint16_t*>(out);
  a.c_t = (int64_t)num_heads * d_v;
  a.c_h = d_v;
  a.pe = nullptr;
  a.pe_t = a.pe_h = 0;
  a.T = tokens;
  a.H = num_heads;
  a.N = d_v;
  a.K = d_latent;
  a.R = 0;
  return launch_rc(mla::launch_absorb_gemm(a, static_cast<hipStream_t>(stream)));
}
int mla_swa_runs(int32_t tokens, int32_t topk, const int32_t* kv_indices,
                 const int32_t* topk_lengths, int32_t page_size, int32_t kv_run_step, int32_t* runs,
                 void* stream) {
  if (tokens < 0 || topk < 1) return MLA_ERR_SHAPE;
  if (!is_pow2(page_size) || page_size > (1 << 30)) return MLA_ERR_PAGE;
  if (kv_run_step != 1 && kv_run_step != -1) return MLA_ERR_MODE;
  if (tokens == 0) return MLA_OK;
  if (kv_indices == nullptr || runs == nullptr) return MLA_ERR_NULL;
  if ((reinterpret_cast<uintptr_t>(kv_indices) & 3u) != 0 || !aligned16(runs) ||
      (topk_lengths != nullptr && (reinterpret_cast<uintptr_t>(topk_lengths) & 3u) != 0))
    return MLA_ERR_ALIGN;
  mla::SwaRunsArgs a;
  a.kv = kv_indices;
  a.lengths = topk_lengths;
  a.runs = runs;
  a.T = tokens;
  a.topk = topk;
  int lg = 0;
  while ((1 << lg) < page_size) ++lg;
  a.ps_log2 = lg;
  a.step = kv_run_step;
  return launch_rc(mla::launch_swa_runs(a, static_cast<hipStream_t>(stream)));
}
int mla_gather_context(const mla_problem* p, int32_t num_reqs, int64_t num_rows,
                       const int32_t* block_table, const int32_t* cu_seq_lens,
                       const int32_t* seq_starts, const int32_t* token_to_seq, const void* kv_cache,
                       void* dst, void* stream) {
  Shape sh;
  int rc = derive(p, 1, &sh);
  if (rc != MLA_OK) return rc;
  if (num_reqs < 1 || num_rows < 0 || num_rows > (int64_t)INT32_MAX * 4) return MLA_ERR_SHAPE;
  if (num_rows == 0) return MLA_OK;
  if (block_table == nullptr || cu_seq_lens == nullptr || token_to_seq == nullptr ||
      kv_cache == nullptr || dst == nullptr)
    return MLA_ERR_NULL;
  if (!aligned16(kv_cache) || !aligned16(dst)) return MLA_ERR_ALIGN;
  mla::GatherArgs a;
  a.cache = static_cast<const uint8_t*>(kv_cache);
  a.block_table = block_table;
  a.cu_seq_lens = cu_seq_lens;
  a.seq_starts = seq_starts;
  a.token_to_seq = token_to_seq;
  a.dst = static_cast<uint16_t*>(dst);
  a.n = num_rows;
  a.page_stride = sh.page_stride;
  a.num_pages = sh.num_pages;
  a.scale_off = (int64_t)sh.page_size * sh.row_bytes;
  a.max_pages = sh.max_pages;
  a.ps_log2 = sh.ps_log2;
  return launch_rc(mla::launch_gather(a, sh.fmt, sh.d_qk, static_cast<hipStream_t>(stream)));
}
int mla_plan_context_chunks(int32_t num_reqs, const int32_t* context_lens, int64_t workspace_rows,
                            int32_t alignment, int32_t max_chunks, int32_t max_spans,
                            int32_t* num_chunks, int32_t* chunk_ptr, int32_t* span_req,
                            int32_t* span_start, int32_t* span_len) {
  if (num_reqs < 0 || alignment < 1 || workspace_rows < alignment || max_chunks < 0 ||
      max_spans < 0)
    return MLA_ERR_SHAPE;
  if (num_chunks == nullptr || chunk_ptr == nullptr || (num_reqs > 0 && context_lens == nullptr))
    return MLA_ERR_NULL;
  int32_t nc = 0, ns = 0;
  int64_t rows = 0;  // rows of the open chunk
  chunk_ptr[0] = 0;
  auto add_span = [&](int32_t r, int64_t start, int64_t len) -> bool {
    if (ns >= max_spans || span_req == nullptr || span_start == nullptr || span_len == nullptr)
      return false;
    span_req[ns] = r;
    span_start[ns] = (int32_t)start;
    span_len[ns] = (int32_t)len;
    ++ns;
    rows += len;
    return true;
  };
  auto close_chunk = [&]() -> bool {
    if (nc >= max_chunks) return false;
    chunk_ptr[++nc] = ns;
    rows = 0;
    return true;
  };
  int64_t s = 0;  // first row of what remains of request r
  for (int32_t r = 0; r < num_reqs;) {
    const int64_t remaining = (int64_t)(context_lens[r] > 0 ? context_lens[r] : 0) - s;
    if (remaining <= 0) {
      ++r;
      s = 0;
      continue;
    }
    if (rows + remaining <= workspace_rows) {  // the whole remainder fits
      if (!add_span(r, s, remaining)) return MLA_ERR_WORKSPACE;
      ++r;
      s = 0;
      if (rows == workspace_rows && !close_chunk()) return MLA_ERR_WORKSPACE;
      continue;
    }
    // the longest aligned prefix that fits, then the chunk is closed
    const int64_t take = (workspace_rows - rows) / alignment * alignment;
    if (take > 0) {
      if (!add_span(r, s, take)) return MLA_ERR_WORKSPACE;
      s += take;
    }
    if (!close_chunk()) return MLA_ERR_WORKSPACE;
  }
  if (rows > 0 && !close_chunk()) return MLA_ERR_WORKSPACE;
  *num_chunks = nc;
  return MLA_OK;
}
const char* mla_build_id(void) { return MLA_BUILD_ID; }

int mla_check_enable(int32_t on) {
  g_checked.store(on != 0, std::memory_order_relaxed);
  return MLA_OK;
}

int mla_check_status(uint32_t* bits, int32_t clear, void* stream) {
  if (bits == nullptr) return MLA_ERR_NULL;
  return mla::check_status(bits, clear != 0, static_cast<hipStream_t>(stream)) == hipSuccess
             ? MLA_OK
             : MLA_ERR_DEVICE;
}

const char* mla_strerror(int status) {
  switch (status) {
    case MLA_OK: return "ok";
    case MLA_ERR_NULL: return "a required pointer is NULL";
    case MLA_ERR_SHAPE: return "unsupported or out-of-range shape";
    case MLA_ERR_FORMAT: return "unknown or unsupported kv_format";
    case MLA_ERR_PAGE: return "invalid page size, page stride or page count";
    case MLA_ERR_MODE: return "unsupported mode combination";
    case MLA_ERR_WORKSPACE: return "workspace buffer too small";
    case MLA_ERR_ALIGN: return "pointer not 16-byte aligned";
    case MLA_ERR_DEVICE: return "HIP device query failed";
    case MLA_ERR_LAUNCH: return "kernel launch failed";
    case MLA_ERR_SCRATCH: return "plan and partials exceed the library's static device scratch";
    default: return "unknown status";
  }
}

}  // extern "C"
