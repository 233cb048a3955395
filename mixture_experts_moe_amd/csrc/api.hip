// C ABI of the fused MoE layer (declared in include/moe.h): argument
// validation, workspace layout, launch policy and kernel timing.  Every
// check runs on the host before the first HIP call.

#include <algorithm>
#include <mutex>
#include <new>
#include <vector>

#include "kernels.h"
#include "moe.h"

// Workspace of moe_forward_noalloc: one array per GPU, in the code object's
// zero-initialised device data, held from module load until the process
// ends.  In host code `scratch` only names the symbol: its device address
// comes from hipGetSymbolAddress, once per device (scratch_address below).
// No `used` attribute: it would keep the device symbol's binding local,
// where the runtime's lookup by name does not find it; referenced from host
// code, the compiler gives it global binding by itself.
static __device__ __align__(256) unsigned char scratch[MOE_NOALLOC_WORKSPACE_BYTES];

namespace {

using moe::FfnArgs;

constexpr int64_t kMaxDim = int64_t(1) << 19;
constexpr int64_t kMaxSlots = int64_t(1) << 30;
constexpr size_t kWsAlign = 256;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

int act_bytes(int dt) { return dt == MOE_DTYPE_F32 ? 4 : 2; }

// ------------------------------------------------------------ validation

int check_desc(const moe_desc* d, int top_k) {
  if (!d) return MOE_ERR_NULL_PTR;
  if (d->act_quant != MOE_ACT_AS_IS && d->act_quant != MOE_ACT_MX_E4M3) return MOE_ERR_BAD_ARG;
  if (d->schedule != MOE_SCHED_AUTO && d->schedule != MOE_SCHED_STATIC &&
      d->schedule != MOE_SCHED_QUEUE)
    return MOE_ERR_BAD_ARG;
  if (d->reserved != 0) return MOE_ERR_BAD_ARG;
  if (d->num_tokens < 0) return MOE_ERR_BAD_SHAPE;
  if (d->hidden < 64 || d->hidden % 64 || d->hidden > kMaxDim) return MOE_ERR_BAD_SHAPE;
  if (d->intermediate < 64 || d->intermediate % 64 || d->intermediate > kMaxDim)
    return MOE_ERR_BAD_SHAPE;
  if (d->num_experts < 1 || d->num_experts > moe::kMaxExperts) return MOE_ERR_BAD_SHAPE;
  if (top_k < 1 || top_k > d->num_experts || top_k > moe::kMaxTopK) return MOE_ERR_BAD_TOPK;
  if (d->num_tokens * top_k >= kMaxSlots) return MOE_ERR_BAD_SHAPE;
  const bool pair_ok = (d->act_dtype == MOE_DTYPE_F32 && d->weight_dtype == MOE_DTYPE_F32) ||
                       (d->act_dtype == MOE_DTYPE_BF16 && d->weight_dtype == MOE_DTYPE_BF16) ||
                       (d->act_dtype == MOE_DTYPE_BF16 && d->weight_dtype == MOE_DTYPE_E4M3FN);
  if (!pair_ok) return MOE_ERR_BAD_DTYPE;
  const int bm = d->block_m;
  if (bm != 0 && bm != 16 && bm != 32 && bm != 64 && bm != 128 && bm != 256)
    return MOE_ERR_BAD_BLOCK_M;
  const int hid = static_cast<int>(d->hidden), inter = static_cast<int>(d->intermediate);
  if (d->act_quant == MOE_ACT_MX_E4M3) {
    // W8A8: bf16 x quantised in the library, e4m3fn weights, the 256-token tile
    if (d->act_dtype != MOE_DTYPE_BF16 || d->weight_dtype != MOE_DTYPE_E4M3FN)
      return MOE_ERR_BAD_DTYPE;
    if (bm != 0 && bm != 256) return MOE_ERR_BAD_BLOCK_M;
    if (!moe::big8_fits(d->num_tokens, hid, inter)) return MOE_ERR_BAD_SHAPE;
    return MOE_OK;
  }
  if (bm == 256 && !(d->weight_dtype == MOE_DTYPE_BF16 &&
                     moe::big_gemm_fits(d->num_tokens, hid, inter)))
    return MOE_ERR_BAD_BLOCK_M;  // the 256-token GEMM is bf16 with d % 256 == 0, I % 128 == 0
  return MOE_OK;
}

int check_scales(const moe_desc* d, const moe_scales* s) {
  if (d->weight_dtype == MOE_DTYPE_E4M3FN) {
    if (!s) return MOE_ERR_NULL_PTR;
    if (s->reserved != 0) return MOE_ERR_BAD_ARG;
    if (s->mode != MOE_SCALE_PER_TENSOR && s->mode != MOE_SCALE_PER_CHANNEL)
      return MOE_ERR_BAD_DTYPE;
    if (!s->w13 || !s->w2) return MOE_ERR_NULL_PTR;
    if (!aligned16(s->w13) || !aligned16(s->w2)) return MOE_ERR_MISALIGNED;
    return MOE_OK;
  }
  if (s && s->mode != MOE_SCALE_NONE) return MOE_ERR_BAD_DTYPE;
  return MOE_OK;
}

int check_ptrs(std::initializer_list<const void*> ptrs) {
  for (const void* p : ptrs)
    if (!p) return MOE_ERR_NULL_PTR;
  for (const void* p : ptrs)
    if (!aligned16(p)) return MOE_ERR_MISALIGNED;
  return MOE_OK;
}

// ------------------------------------------------------------ launch plan

struct Plan {
  int T, d, E, I, k, A, B, cap;
  int splits, ksplit;
  int act, wdt;
  bool act_mx;  // W8A8 mode
  bool queue;   // tile-queue schedule of the 128-token GEMM
  bool wide;    // blocks of 128 on the register-token tile (automatic schedule)
  // workspace offsets (bytes); xq, sx, sh only in the W8A8 mode, qcnt only
  // with the queue schedule
  size_t logits, ids, gates, counts, num_padded, sorted, block_exp, h, y, xq, sx, sh, qcnt, total;
  size_t rpart;  // the split router's partial tiles (layer path, few tokens), or the
                 // LDS-staged router's quarter logits (many tokens and experts), or 0
  bool rsplit;
  bool rlds;
  bool fused;    // W13, W2 and combine as one persistent launch (layer path, decode)
  bool w2c;      // W2 with the combine in its launch (layer path, decode)
  size_t fcnt;   // counters of either, cleared by the routing launch
  int nfcnt;
};

// Block size of the regrouped layout.  Up to 64 tokens the weight-streaming
// kernels mostly run with B >= T: every expert's tokens fit one block (an
// expert holds at most one slot per token), so each expert's weights are
// streamed exactly once; where experts average few slots (at most 8 with
// bf16 weights, 4 with e4m3fn) blocks of 16, an expert holding more taking
// further blocks.  Larger batches use 128-token blocks (the register-token
// tile, else the token-tiled grouped GEMM), and when experts average 256
// tokens or more (bf16 weights, fitting shapes) 256-token blocks and the
// large-tile GEMM.
int default_block_m(const moe_desc* d, int top_k) {
  if (d->act_quant == MOE_ACT_MX_E4M3) return 256;  // the W8A8 tile
  if (d->weight_dtype == MOE_DTYPE_F32) return 16;
  const int64_t T = d->num_tokens;
  const int hid = static_cast<int>(d->hidden), inter = static_cast<int>(d->intermediate);
  const bool bf16_act = d->act_dtype == MOE_DTYPE_BF16;
  if (T <= 16) return 16;
  // e4m3fn weights with experts averaging at most 4 slots: blocks of 16 keep
  // the LDS-streaming kernel (an expert holding more takes further blocks)
  if (T <= 64 && d->weight_dtype == MOE_DTYPE_E4M3FN && bf16_act &&
      T * top_k <= 4 * d->num_experts && moe::dma_stream_fits(hid, inter, MOE_DTYPE_E4M3FN))
    return 16;
  // bf16 weights with experts averaging at most 8 slots (the decode shape
  // at T = 32: 287 -> 279 us for W13 against blocks of 32, whose second
  // token subtile is mostly padding); at 16 slots (T = 64) an expert's
  // second block of 16 re-reads its weights and blocks of 32 win
  if (T <= 64 && d->weight_dtype == MOE_DTYPE_BF16 && bf16_act &&
      T * top_k <= 8 * d->num_experts && moe::dma_stream_fits(hid, inter, MOE_DTYPE_BF16))
    return 16;
  if (T <= 32) return 32;
  if (T <= 64) {
    // blocks of 32 keep the LDS-streaming kernel (an expert holding more
    // than 32 of the tokens takes a second block)
    const bool lds = d->weight_dtype == MOE_DTYPE_BF16 && bf16_act &&
                     moe::dma_stream_fits(hid, inter, MOE_DTYPE_BF16);
    return lds ? 32 : 64;
  }
  const int64_t per_expert = T * top_k / d->num_experts;
  if (per_expert >= 256 && d->weight_dtype == MOE_DTYPE_BF16 &&
      moe::big_gemm_fits(d->num_tokens, static_cast<int>(d->hidden), static_cast<int>(d->intermediate)))
    return 256;
  return 128;
}

// W2 K split for blocks of <= 64 tokens: double the splits while the grid
// has fewer waves than this, each split keeps at least this many K chunks,
// and there are fewer splits than the maximum.
#ifndef MOE_W2_SPLIT_WAVES
#define MOE_W2_SPLIT_WAVES 2048
#endif
#ifndef MOE_W2_MIN_CHUNKS
#define MOE_W2_MIN_CHUNKS 4
#endif
// (Four, not eight: the decode shape at T = 1, two experts, reached eight
// splits of seven stages each and spent more on starting them; W2 with the
// combine 49.7 -> 43.3 us, the other decode batches unchanged.)
#ifndef MOE_W2_MAX_SPLITS
#define MOE_W2_MAX_SPLITS 4
#endif

// Big-tile W2 K split: double the splits while the grid has fewer
// workgroups than this and there are fewer splits than the maximum.
#ifndef MOE_BIG_W2_SPLIT_WGS
#define MOE_BIG_W2_SPLIT_WGS 1024
#endif
#ifndef MOE_BIG_W2_MAX_SPLITS
#define MOE_BIG_W2_MAX_SPLITS 4
#endif

// Register-token tile W2 K split: double the splits while the grid has
// fewer workgroups than this, there are fewer splits than the maximum, and
// each range keeps at least the minimum number of K stages.
#ifndef MOE_WIDE_W2_SPLIT_WGS
#define MOE_WIDE_W2_SPLIT_WGS 1024
#endif
#ifndef MOE_WIDE_W2_MAX_SPLITS
#define MOE_WIDE_W2_MAX_SPLITS 4
#endif
// (32, not 8: at the skew shape, I = 2880, two ranges of 22 stages cost
// more in ring fill and in the combine's second set of partials than they
// gained in grid fill, W2 + combine 138 -> 129 us; the decode shapes at
// T = 128..1024, I = 14336, keep their splits.)
#ifndef MOE_WIDE_W2_MIN_STAGES
#define MOE_WIDE_W2_MIN_STAGES 32
#endif

int64_t capacity(int64_t A, int64_t E, int64_t B) {
  const int64_t n = A + (E < A ? E : A) * (B - 1);
  return (n + B - 1) / B * B;
}

void make_plan(const moe_desc* d, int top_k, bool with_routing, Plan* p) {
  p->T = static_cast<int>(d->num_tokens);
  p->d = static_cast<int>(d->hidden);
  p->E = static_cast<int>(d->num_experts);
  p->I = static_cast<int>(d->intermediate);
  p->k = top_k;
  p->A = p->T * top_k;
  p->B = d->block_m ? d->block_m : default_block_m(d, top_k);
  p->cap = static_cast<int>(capacity(p->A, p->E, p->B));
  p->act = d->act_dtype;
  p->wdt = d->weight_dtype;
  p->act_mx = d->act_quant == MOE_ACT_MX_E4M3;
  // blocks of 128: the register-token tile where it fits, unless the caller
  // asked for one of the 128-token GEMM's schedules
  p->wide = d->schedule == MOE_SCHED_AUTO &&
            moe::wide_use(p->wdt, p->act, p->act_mx, p->B, p->T, p->d, p->I);
  p->queue = d->schedule != MOE_SCHED_STATIC && p->B == 128 && p->wdt != MOE_DTYPE_F32 &&
             !p->act_mx && !p->wide;

  // Split W2's K range when there are too few workgroups to keep enough
  // HBM requests in flight (small batches); the combine adds the splits in a
  // fixed order.
  p->splits = 1;
  p->ksplit = p->I;
  if (p->A > 0 && p->B == 256) {
    // the big-tile W2 has d/256 channel tiles per block: split K until the
    // grid fills about four rounds of the CUs (splits of >= 16 stages)
    const int64_t blocks_est = moe::ffn_blocks_estimate(p->cap, p->B, p->E, p->A);
    const int64_t tiles = blocks_est * (p->d / 256);
    const int kc = p->act_mx ? moe::big8_w2_kchunk() : moe::big_w2_kchunk();
    int s = 1;
    while (s < MOE_BIG_W2_MAX_SPLITS && tiles * s < MOE_BIG_W2_SPLIT_WGS &&
           p->I / (2 * s) >= 8 * kc)
      s *= 2;
#ifdef MOE_BIG_W2_SPLITS
    s = MOE_BIG_W2_SPLITS;
#endif
    const int per = (p->I + s - 1) / s;
    p->ksplit = (per + kc - 1) / kc * kc;
    p->splits = (p->I + p->ksplit - 1) / p->ksplit;
  }
  if (p->A > 0 && p->wide) {
    // the register-token tile's W2 has ceil(d/256) channel tiles per block:
    // split K until the grid fills about four rounds of the CUs, each range
    // keeping at least MOE_WIDE_W2_MIN_STAGES stages
    const int64_t blocks_est = moe::ffn_blocks_estimate(p->cap, p->B, p->E, p->A);
    const int64_t tiles = blocks_est * ((p->d + 255) / 256);
    const int kc = moe::wide_kchunk(p->wdt);
    int s = 1;
    while (s < MOE_WIDE_W2_MAX_SPLITS && tiles * s < MOE_WIDE_W2_SPLIT_WGS &&
           p->I / (2 * s) >= MOE_WIDE_W2_MIN_STAGES * kc)
      s *= 2;
    // every range, the last included, keeps at least the minimum (the
    // tile's ring needs a few stages)
    int per = (p->I + s - 1) / s;
    per = (per + kc - 1) / kc * kc;
    while (s > 1 && p->I - (p->I + per - 1) / per * per + per < MOE_WIDE_W2_MIN_STAGES * kc) {
      s /= 2;
      per = ((p->I + s - 1) / s + kc - 1) / kc * kc;
    }
    p->ksplit = per;
    p->splits = (p->I + p->ksplit - 1) / p->ksplit;
  } else if (p->wdt != MOE_DTYPE_F32 && p->A > 0 && p->B <= 64) {  // the 128-token GEMM does not split
    const int64_t blocks_est = moe::ffn_blocks_estimate(p->cap, p->B, p->E, p->A);
    const bool lds = moe::dma_stream_use(p->wdt, p->act, p->B, p->d, p->I, blocks_est);
    const int kc = moe::ffn2_kchunk(p->d, p->I, p->B, p->wdt, p->act, blocks_est);
    // one wave per dma_w2_channels() (LDS streaming) or about 32 (register
    // path) output channels
    const int64_t waves =
        blocks_est * (p->d / (lds ? moe::dma_w2_channels(p->wdt, p->B, blocks_est) : 32));
    int s = 1;
    while (s < MOE_W2_MAX_SPLITS && waves * s < MOE_W2_SPLIT_WAVES &&
           p->I / (2 * s) >= MOE_W2_MIN_CHUNKS * kc)
      s *= 2;
    const int per = (p->I + s - 1) / s;
    p->ksplit = (per + kc - 1) / kc * kc;
    p->splits = (p->I + p->ksplit - 1) / p->ksplit;
  }

  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = round_up(off + bytes, kWsAlign);
    return at;
  };
  const size_t T = p->T, E = p->E, A = p->A, cap = p->cap;
  if (with_routing) {
    p->logits = take(T * E * 4);
    p->ids = take(A * 4);
    p->gates = take(A * 4);
    p->counts = take(E * 4);
    p->num_padded = take(4);
    p->sorted = take(cap * 4);
    p->block_exp = take(cap / p->B * 4);
  } else {
    p->rsplit = false;
    p->rlds = false;
    p->rpart = 0;
    p->logits = p->ids = p->gates = p->counts = p->num_padded = p->sorted = p->block_exp = 0;
  }
  // h: bf16 (fp32 for fp32 layers), or e4m3fn codes in the W8A8 mode
  p->h = take(cap * static_cast<size_t>(p->I) * (p->act_mx ? 1 : act_bytes(p->act)));
  p->y = take(static_cast<size_t>(p->splits) * A * p->d * 4);
  if (p->act_mx) {
    p->xq = take(T * static_cast<size_t>(p->d));
    p->sx = take(T * static_cast<size_t>(p->d) / 32);
    p->sh = take(cap * static_cast<size_t>(p->I) / 32);
  } else {
    p->xq = p->sx = p->sh = 0;
  }
  p->qcnt = p->queue ? take(moe::gemm_queue_ints() * 4) : 0;
  p->fused = false;
  p->w2c = false;
  p->fcnt = 0;
  p->nfcnt = 0;
  if (with_routing) {
    p->rsplit = moe::router_fused(p->act, p->T, p->E) ||
                moe::router_split_logits(p->act, p->T, p->E);
    p->rlds = !p->rsplit && moe::router_lds_logits(p->act, p->T, p->E, p->d);
    p->rpart = p->rsplit ? take(moe::router_split_bytes(p->T, p->E))
               : p->rlds ? take(moe::router_lds_bytes(p->T, p->E))
                         : 0;
    // the fused decode kernel: its counters are cleared by the split
    // router's first launch, so it runs where that launch does
    const int64_t blocks_est = moe::ffn_blocks_estimate(p->cap, p->B, p->E, p->A);
    if (p->rsplit && p->A > 0 && d->schedule == MOE_SCHED_QUEUE && !p->act_mx &&
        moe::fused_decode_fits(p->wdt, p->act, p->B, p->d, p->I, blocks_est)) {
      FfnArgs a{};
      a.T = p->T;
      a.d = p->d;
      a.E = p->E;
      a.I = p->I;
      a.A = p->A;
      a.B = p->B;
      a.cap = p->cap;
      a.splits = p->splits;
      a.w_dtype = p->wdt;
      p->nfcnt = moe::fused_counter_ints(a);
      p->fcnt = take(static_cast<size_t>(p->nfcnt) * 4);
      p->fused = true;
    } else if (p->rsplit && p->A > 0 && d->schedule == MOE_SCHED_AUTO && !p->act_mx &&
               p->act == MOE_DTYPE_BF16 &&
               moe::dma_stream_use(p->wdt, p->act, p->B, p->d, p->I, blocks_est) &&
               moe::ffn2_combine_pays(p->wdt, p->B, blocks_est) &&
               p->d % moe::dma_w2_channels(p->wdt, p->B, blocks_est) == 0) {
      FfnArgs a{};
      a.T = p->T;
      a.d = p->d;
      a.E = p->E;
      a.A = p->A;
      a.B = p->B;
      a.cap = p->cap;
      a.w_dtype = p->wdt;
      p->nfcnt = moe::ffn2_combine_ints(a);
      p->fcnt = take(static_cast<size_t>(p->nfcnt) * 4);
      p->w2c = true;
    }
  }
  p->total = p->T == 0 ? 0 : off;  // nothing runs for T = 0
}

// ------------------------------------------------------------ timing

struct Pending {
  int kind;
  hipEvent_t start, stop;
};

std::mutex g_timing_mu;
uint32_t g_timing_mask = 0;  // bit k: time kernels of kind k
std::vector<Pending> g_pending;
std::vector<std::pair<hipEvent_t, hipEvent_t>> g_event_pool;
double g_total_ms[MOE_KERNEL_COUNT] = {};
int64_t g_launches[MOE_KERNEL_COUNT] = {};

// Set while this thread records a graph: captured launches are not timed.
thread_local bool t_capturing = false;

template <class F>
hipError_t timed(int kind, hipStream_t s, F&& launch) {
  bool on;
  {
    std::lock_guard<std::mutex> lk(g_timing_mu);
    on = (g_timing_mask >> kind) & 1u;
  }
  if (!on || t_capturing) return launch();
  hipEvent_t a, b;
  {
    std::lock_guard<std::mutex> lk(g_timing_mu);
    if (!g_event_pool.empty()) {
      a = g_event_pool.back().first;
      b = g_event_pool.back().second;
      g_event_pool.pop_back();
    } else {
      if (hipEventCreate(&a) != hipSuccess) return hipErrorOutOfMemory;
      if (hipEventCreate(&b) != hipSuccess) {
        (void)hipEventDestroy(a);
        return hipErrorOutOfMemory;
      }
    }
  }
  hipError_t err = hipEventRecord(a, s);
  if (err == hipSuccess) err = launch();
  if (err == hipSuccess) err = hipEventRecord(b, s);
  std::lock_guard<std::mutex> lk(g_timing_mu);
  if (err == hipSuccess)
    g_pending.push_back({kind, a, b});
  else
    g_event_pool.push_back({a, b});
  return err;
}

// ------------------------------------------------------------ launch sequences

int to_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

FfnArgs ffn_args(const Plan& p, const void* x, const void* w13, const void* w2,
                 const moe_scales* sc, const float* topk_w, const int32_t* sorted,
                 const int32_t* block_exp, const int32_t* num_padded, void* out, char* ws) {
  FfnArgs a{};
  a.x = x;
  a.w13 = w13;
  a.w2 = w2;
  const bool fp8 = p.wdt == MOE_DTYPE_E4M3FN;
  a.s13 = fp8 ? sc->w13 : nullptr;
  a.s2 = fp8 ? sc->w2 : nullptr;
  a.scale_mode = fp8 ? sc->mode : moe::kScaleNone;
  a.act_dtype = p.act;
  a.w_dtype = p.wdt;
  a.topk_w = topk_w;
  a.sorted_ids = sorted;
  a.block_expert = block_exp;
  a.num_padded = num_padded;
  a.h = ws + p.h;
  a.y_part = reinterpret_cast<float*>(ws + p.y);
  a.out = out;
  a.T = p.T;
  a.d = p.d;
  a.E = p.E;
  a.I = p.I;
  a.k = p.k;
  a.A = p.A;
  a.B = p.B;
  a.cap = p.cap;
  a.splits = p.splits;
  a.ksplit = p.ksplit;
  a.act_mx = p.act_mx;
  a.xq = p.act_mx ? reinterpret_cast<uint8_t*>(ws + p.xq) : nullptr;
  a.sx = p.act_mx ? reinterpret_cast<uint8_t*>(ws + p.sx) : nullptr;
  a.sh = p.act_mx ? reinterpret_cast<uint8_t*>(ws + p.sh) : nullptr;
  a.queue_sched = p.queue;
  a.queue = p.queue ? reinterpret_cast<int32_t*>(ws + p.qcnt) : nullptr;
  a.wide = p.wide;
  return a;
}

hipError_t run_ffn(const FfnArgs& a, hipStream_t s) {
  if (a.fused_cnt)  // W13, W2 and the combine in one persistent launch
    return timed(MOE_KERNEL_FFN_FUSED, s, [&] { return moe::launch_ffn_fused(a, s); });
  hipError_t e = hipSuccess;
  if (a.act_mx) e = timed(MOE_KERNEL_QUANT_X, s, [&] { return moe::launch_quantize_x(a, s); });
  if (e == hipSuccess && a.queue_sched && !a.queue_zeroed) e = moe::launch_gemm_queue_reset(a, s);
  if (e == hipSuccess) e = timed(MOE_KERNEL_FFN13, s, [&] { return moe::launch_ffn13(a, s); });
  if (e == hipSuccess && a.combine_cnt)  // W2 adds up each token's slots itself
    return timed(MOE_KERNEL_FFN2, s, [&] { return moe::launch_ffn2_combine_dma(a, s); });
  if (e == hipSuccess) e = timed(MOE_KERNEL_FFN2, s, [&] { return moe::launch_ffn2(a, s); });
  if (e == hipSuccess) e = timed(MOE_KERNEL_COMBINE, s, [&] { return moe::launch_combine(a, s); });
  return e;
}

}  // namespace

extern "C" {

MOE_API const char* moe_strerror(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_NULL_PTR: return "a required pointer is NULL";
    case MOE_ERR_BAD_SHAPE: return "bad shape (d and I must be multiples of 64 in [64, 2^19], 1 <= E <= 1024, T >= 0, T*top_k < 2^30)";
    case MOE_ERR_BAD_TOPK: return "top_k must be in [1, min(E, 64)]";
    case MOE_ERR_BAD_DTYPE: return "unsupported dtype pair or scale mode (supported: f32/f32, bf16/bf16, bf16/e4m3fn with per-tensor or per-channel scales)";
    case MOE_ERR_MISALIGNED: return "a pointer is not 16-byte aligned (workspace: 256-byte)";
    case MOE_ERR_WORKSPACE: return "workspace is NULL or smaller than moe_workspace_bytes()";
    case MOE_ERR_HIP: return "a HIP call or kernel launch failed";
    case MOE_ERR_BAD_BLOCK_M: return "block_m must be 0, 16, 32, 64, 128 or 256 (256: bf16 weights, d % 256 == 0, I % 128 == 0, 4*I*d and 2*T*d under 2^31)";
    case MOE_ERR_BAD_ARG: return "invalid argument (reserved fields must be 0)";
    case MOE_ERR_NOALLOC_SIZE: return "the layer needs more workspace than moe_forward_noalloc's static array (MOE_NOALLOC_WORKSPACE_BYTES, 64 MiB); call moe_forward with a caller workspace";
  }
  return "unknown status";
}

MOE_API int moe_align_capacity(const moe_desc* desc, int top_k, int32_t* block_m,
                               int64_t* cap) {
  int st = check_desc(desc, top_k);
  if (st) return st;
  if (!block_m || !cap) return MOE_ERR_NULL_PTR;
  Plan p;
  make_plan(desc, top_k, true, &p);
  *block_m = p.B;
  *cap = p.cap;
  return MOE_OK;
}

MOE_API int moe_workspace_bytes(const moe_desc* desc, int top_k, int with_routing,
                                size_t* bytes) {
  int st = check_desc(desc, top_k);
  if (st) return st;
  if (!bytes) return MOE_ERR_NULL_PTR;
  Plan p;
  make_plan(desc, top_k, with_routing != 0, &p);
  *bytes = p.total;
  return MOE_OK;
}

// Router logits and top-k: one kernel when the router kernel can select
// itself (timed as route_logits), else two launches.
// `part` (or nullptr): scratch for the split router when it applies.
// `zero`, `nzero`: counters the split router's first launch clears (only
// with `part`).
static hipError_t route(const void* x, int act, const float* w_gate, float* logits,
                        int32_t* ids, float* gates, int T, int E, int d, int k, void* part,
                        hipStream_t s, int32_t* zero = nullptr, int nzero = 0) {
  if (moe::router_fused(act, T, E))
    return timed(MOE_KERNEL_ROUTE_LOGITS, s, [&] {
      return part ? moe::launch_router_fused_split(x, w_gate, logits, ids, gates, T, E, d, k,
                                                   part, s, zero, nzero)
                  : moe::launch_router_fused(x, w_gate, logits, ids, gates, T, E, d, k, s);
    });
  if (moe::router_selects(act, T, E))  // at most 16 experts: the logits kernel selects too
    return timed(MOE_KERNEL_ROUTE_LOGITS, s, [&] {
      return moe::launch_router_fused(x, w_gate, logits, ids, gates, T, E, d, k, s);
    });
  if (part && moe::router_lds_logits(act, T, E, d))  // logits, then selection with the sum
    return timed(MOE_KERNEL_ROUTE_LOGITS, s, [&] {
      return moe::launch_router_lds_topk(x, w_gate, logits, ids, gates, T, E, d, k, part, s);
    });
  hipError_t e = timed(MOE_KERNEL_ROUTE_LOGITS, s, [&] {
    return part && moe::router_split_logits(act, T, E)
               ? moe::launch_router_split_logits(x, w_gate, logits, T, E, d, part, s, zero,
                                                 nzero)
               : moe::launch_router_logits(x, act, w_gate, logits, T, E, d, s);
  });
  if (e == hipSuccess)
    e = timed(MOE_KERNEL_ROUTE_TOPK, s,
              [&] { return moe::launch_router_topk(logits, ids, gates, T, E, k, s); });
  return e;
}

// Routing followed by the regrouping: the router's single workgroup also
// regroups when it can (timed as route_logits), else route() then the
// regrouping kernel.  `part` (or nullptr): scratch for the split router.
// `queue` (or nullptr): the expert kernels' work-queue counters;
// *queue_zeroed tells whether the align launch has cleared them.
static hipError_t route_align(const Plan& p, const void* x, const float* w_gate, float* logits,
                              int32_t* ids, float* gates, int32_t* counts, int32_t* sorted,
                              int32_t* block_exp, int32_t* num_padded, void* part,
                              int32_t* queue, bool* queue_zeroed, hipStream_t s,
                              int32_t* fcnt = nullptr) {
  *queue_zeroed = false;
  const int nf = fcnt ? p.nfcnt : 0;
  if (moe::route_align_fused(p.act, p.T, p.E))
    return timed(MOE_KERNEL_ROUTE_LOGITS, s, [&] {
      return part ? moe::launch_route_align_fused_split(x, w_gate, logits, ids, gates, p.T, p.E,
                                                        p.d, p.k, p.B, p.cap, counts, sorted,
                                                        block_exp, num_padded, part, s, fcnt,
                                                        nf)
                  : moe::launch_route_align_fused(x, w_gate, logits, ids, gates, p.T, p.E, p.d,
                                                  p.k, p.B, p.cap, counts, sorted, block_exp,
                                                  num_padded, s);
    });
  hipError_t e =
      route(x, p.act, w_gate, logits, ids, gates, p.T, p.E, p.d, p.k, part, s, fcnt, nf);
  const int nzero = queue ? moe::gemm_queue_ints() : 0;
  if (e == hipSuccess)
    e = timed(MOE_KERNEL_ALIGN, s, [&] {
      return moe::launch_align(ids, p.A, p.E, p.B, p.cap, counts, sorted, block_exp, num_padded, s,
                               queue, nzero);
    });
  *queue_zeroed = e == hipSuccess && nzero > 0;
  return e;
}

MOE_API int moe_route(const moe_desc* desc, const void* x, const float* w_gate, int top_k,
                      float* logits, int32_t* topk_ids, float* topk_w, void* stream) {
  int st = check_desc(desc, top_k);
  if (st) return st;
  const int T = static_cast<int>(desc->num_tokens);
  if (T == 0) return MOE_OK;
  if ((st = check_ptrs({x, w_gate, logits, topk_ids, topk_w}))) return st;
  const int E = static_cast<int>(desc->num_experts), d = static_cast<int>(desc->hidden);
  hipStream_t s = static_cast<hipStream_t>(stream);
  return to_status(
      route(x, desc->act_dtype, w_gate, logits, topk_ids, topk_w, T, E, d, top_k, nullptr, s));
}

MOE_API int moe_route_logits(const moe_desc* desc, const float* logits, int top_k,
                             int32_t* topk_ids, float* topk_w, void* stream) {
  int st = check_desc(desc, top_k);
  if (st) return st;
  const int T = static_cast<int>(desc->num_tokens);
  if (T == 0) return MOE_OK;
  if ((st = check_ptrs({logits, topk_ids, topk_w}))) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return to_status(timed(MOE_KERNEL_ROUTE_TOPK, s, [&] {
    return moe::launch_router_topk(logits, topk_ids, topk_w, T,
                                   static_cast<int>(desc->num_experts), top_k, s);
  }));
}

MOE_API int moe_align(const moe_desc* desc, const int32_t* topk_ids, int top_k, int32_t* counts,
                      int32_t* sorted_ids, int32_t* block_expert, int32_t* num_padded,
                      void* stream) {
  int st = check_desc(desc, top_k);
  if (st) return st;
  if (desc->num_tokens == 0) return MOE_OK;
  if ((st = check_ptrs({topk_ids, counts, sorted_ids, block_expert, num_padded}))) return st;
  Plan p;
  make_plan(desc, top_k, true, &p);
  hipStream_t s = static_cast<hipStream_t>(stream);
  return to_status(timed(MOE_KERNEL_ALIGN, s, [&] {
    return moe::launch_align(topk_ids, p.A, p.E, p.B, p.cap, counts, sorted_ids, block_expert,
                             num_padded, s);
  }));
}

MOE_API int moe_route_align(const moe_desc* desc, const void* x, const float* w_gate, int top_k,
                            float* logits, int32_t* topk_ids, float* topk_w, int32_t* counts,
                            int32_t* sorted_ids, int32_t* block_expert, int32_t* num_padded,
                            void* stream) {
  int st = check_desc(desc, top_k);
  if (st) return st;
  if (desc->num_tokens == 0) return MOE_OK;
  if ((st = check_ptrs({x, w_gate, logits, topk_ids, topk_w, counts, sorted_ids, block_expert,
                        num_padded})))
    return st;
  Plan p;
  make_plan(desc, top_k, true, &p);
  hipStream_t s = static_cast<hipStream_t>(stream);
  bool zeroed = false;
  return to_status(route_align(p, x, w_gate, logits, topk_ids, topk_w, counts, sorted_ids,
                               block_expert, num_padded, nullptr, nullptr, &zeroed, s));
}

MOE_API int moe_expert_ffn(const moe_desc* desc, const void* x, const void* w13, const void* w2,
                           int top_k, const moe_scales* scales, const float* topk_w,
                           const int32_t* sorted_ids, const int32_t* block_expert,
                           const int32_t* num_padded, void* out, void* workspace,
                           size_t workspace_bytes, void* stream) {
  int st = check_desc(desc, top_k);
  if (st) return st;
  if (desc->num_tokens == 0) return MOE_OK;
  if ((st = check_scales(desc, scales))) return st;
  if ((st = check_ptrs({x, w13, w2, topk_w, sorted_ids, block_expert, num_padded, out})))
    return st;
  Plan p;
  make_plan(desc, top_k, false, &p);
  if (!workspace || workspace_bytes < p.total) return MOE_ERR_WORKSPACE;
  if (reinterpret_cast<uintptr_t>(workspace) % kWsAlign) return MOE_ERR_MISALIGNED;
  char* ws = static_cast<char*>(workspace);
  hipStream_t s = static_cast<hipStream_t>(stream);
  FfnArgs a = ffn_args(p, x, w13, w2, scales, topk_w, sorted_ids, block_expert, num_padded, out,
                       ws);
  return to_status(run_ffn(a, s));
}

MOE_API int moe_quantize_act(const moe_desc* desc, const void* x, uint8_t* codes, uint8_t* exps,
                             void* stream) {
  int st = check_desc(desc, 1);
  if (st) return st;
  if (desc->act_quant != MOE_ACT_MX_E4M3) return MOE_ERR_BAD_ARG;
  if (desc->num_tokens == 0) return MOE_OK;
  if ((st = check_ptrs({x, codes, exps}))) return st;
  FfnArgs a{};
  a.x = x;
  a.T = static_cast<int>(desc->num_tokens);
  a.d = static_cast<int>(desc->hidden);
  a.act_mx = true;
  a.xq = codes;
  a.sx = exps;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return to_status(timed(MOE_KERNEL_QUANT_X, s, [&] { return moe::launch_quantize_x(a, s); }));
}

// Checks shared by moe_forward and moe_graph_create; fills the plan.
static int forward_checks(const moe_desc* desc, const void* x, const float* w_gate,
                          const void* w13, const void* w2, int top_k, const moe_scales* scales,
                          void* out, void* workspace, size_t workspace_bytes, Plan* p) {
  int st = check_desc(desc, top_k);
  if (st) return st;
  if (desc->num_tokens == 0) return MOE_OK;
  if ((st = check_scales(desc, scales))) return st;
  if ((st = check_ptrs({x, w_gate, w13, w2, out}))) return st;
  make_plan(desc, top_k, true, p);
  if (!workspace || workspace_bytes < p->total) return MOE_ERR_WORKSPACE;
  if (reinterpret_cast<uintptr_t>(workspace) % kWsAlign) return MOE_ERR_MISALIGNED;
  return MOE_OK;
}

// The whole layer on stream s (T > 0, arguments checked).
static int enqueue_forward(const Plan& p, const void* x, const float* w_gate, const void* w13,
                           const void* w2, const moe_scales* scales, void* out, char* ws,
                           hipStream_t s) {
  float* logits = reinterpret_cast<float*>(ws + p.logits);
  int32_t* ids = reinterpret_cast<int32_t*>(ws + p.ids);
  float* gates = reinterpret_cast<float*>(ws + p.gates);
  int32_t* counts = reinterpret_cast<int32_t*>(ws + p.counts);
  int32_t* num_padded = reinterpret_cast<int32_t*>(ws + p.num_padded);
  int32_t* sorted = reinterpret_cast<int32_t*>(ws + p.sorted);
  int32_t* block_exp = reinterpret_cast<int32_t*>(ws + p.block_exp);

  int32_t* queue = p.queue ? reinterpret_cast<int32_t*>(ws + p.qcnt) : nullptr;
  int32_t* fcnt = p.fused || p.w2c ? reinterpret_cast<int32_t*>(ws + p.fcnt) : nullptr;
  bool zeroed = false;
  void* part = p.rsplit || p.rlds ? ws + p.rpart : nullptr;
  const hipError_t e = route_align(p, x, w_gate, logits, ids, gates, counts, sorted, block_exp,
                                   num_padded, part, queue, &zeroed, s, fcnt);
  if (e != hipSuccess) return MOE_ERR_HIP;
  FfnArgs a = ffn_args(p, x, w13, w2, scales, gates, sorted, block_exp, num_padded, out, ws);
  a.queue_zeroed = zeroed;
  a.fused_cnt = p.fused ? fcnt : nullptr;
  a.combine_cnt = p.w2c ? fcnt : nullptr;
  return to_status(run_ffn(a, s));
}

// Device address of `scratch` on the device that runs `stream` (the current
// device for the null stream), fetched with that device current on the first
// call for it and kept per device.
constexpr int kMaxScratchDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_addr[kMaxScratchDevices] = {};

static int scratch_address(hipStream_t stream, void** addr) {
  int cur = 0;
  if (hipGetDevice(&cur) != hipSuccess) return MOE_ERR_HIP;
  int dev = cur;
  if (stream) {
    hipDevice_t sd;
    if (hipStreamGetDevice(stream, &sd) != hipSuccess) return MOE_ERR_HIP;
    dev = static_cast<int>(sd);
  }
  if (dev < 0 || dev >= kMaxScratchDevices) return MOE_ERR_HIP;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_addr[dev]) {
    if (dev != cur && hipSetDevice(dev) != hipSuccess) return MOE_ERR_HIP;
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (dev != cur && hipSetDevice(cur) != hipSuccess) return MOE_ERR_HIP;
    if (e != hipSuccess || !p) return MOE_ERR_HIP;
    g_scratch_addr[dev] = p;
  }
  *addr = g_scratch_addr[dev];
  return MOE_OK;
}

MOE_API int moe_forward(const moe_desc* desc, const void* x, const float* w_gate,
                        const void* w13, const void* w2, int top_k, const moe_scales* scales,
                        void* out, void* workspace, size_t workspace_bytes, void* stream) {
  Plan p;
  const int st = forward_checks(desc, x, w_gate, w13, w2, top_k, scales, out, workspace,
                                workspace_bytes, &p);
  if (st || desc->num_tokens == 0) return st;
  return enqueue_forward(p, x, w_gate, w13, w2, scales, out, static_cast<char*>(workspace),
                         static_cast<hipStream_t>(stream));
}

MOE_API int moe_forward_noalloc(const moe_desc* desc, const void* x, const float* w_gate,
                                const void* w13, const void* w2, int top_k,
                                const moe_scales* scales, void* out, void* stream) {
  int st = check_desc(desc, top_k);
  if (st) return st;
  if (desc->num_tokens == 0) return MOE_OK;
  if ((st = check_scales(desc, scales))) return st;
  if ((st = check_ptrs({x, w_gate, w13, w2, out}))) return st;
  Plan p;
  make_plan(desc, top_k, true, &p);
  if (p.total > static_cast<size_t>(MOE_NOALLOC_WORKSPACE_BYTES)) return MOE_ERR_NOALLOC_SIZE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  void* ws = nullptr;
  if ((st = scratch_address(s, &ws))) return st;
  // every region the layer reads is written earlier in the same call (the
  // align launch clears the queue counters), as with a caller workspace
  return enqueue_forward(p, x, w_gate, w13, w2, scales, out, static_cast<char*>(ws), s);
}

}  // extern "C"

// Opaque graph handle: the instantiated graph (NULL for T = 0, whose
// replay does nothing).
struct moe_graph {
  hipGraphExec_t exec;
};

extern "C" {

MOE_API int moe_graph_create(const moe_desc* desc, const void* x, const float* w_gate,
                             const void* w13, const void* w2, int top_k,
                             const moe_scales* scales, void* out, void* workspace,
                             size_t workspace_bytes, moe_graph** graph) {
  if (!graph) return MOE_ERR_NULL_PTR;
  *graph = nullptr;
  Plan p;
  int st = forward_checks(desc, x, w_gate, w13, w2, top_k, scales, out, workspace,
                          workspace_bytes, &p);
  if (st) return st;
  if (desc->num_tokens == 0) {
    *graph = new (std::nothrow) moe_graph{nullptr};
    return *graph ? MOE_OK : MOE_ERR_HIP;
  }
  // record on a private stream; thread-local capture mode leaves other
  // threads' HIP calls alone
  hipStream_t cs;
  if (hipStreamCreateWithFlags(&cs, hipStreamNonBlocking) != hipSuccess) return MOE_ERR_HIP;
  hipGraph_t g = nullptr;
  if (hipStreamBeginCapture(cs, hipStreamCaptureModeThreadLocal) != hipSuccess) {
    (void)hipStreamDestroy(cs);
    return MOE_ERR_HIP;
  }
  t_capturing = true;
  st = enqueue_forward(p, x, w_gate, w13, w2, scales, out, static_cast<char*>(workspace), cs);
  t_capturing = false;
  const hipError_t ce = hipStreamEndCapture(cs, &g);  // always ends the capture
  (void)hipStreamDestroy(cs);
  if (st == MOE_OK && (ce != hipSuccess || !g)) st = MOE_ERR_HIP;
  hipGraphExec_t exec = nullptr;
  if (st == MOE_OK && hipGraphInstantiate(&exec, g, nullptr, nullptr, 0) != hipSuccess)
    st = MOE_ERR_HIP;
  if (g) (void)hipGraphDestroy(g);
  if (st != MOE_OK) return st;
  *graph = new (std::nothrow) moe_graph{exec};
  if (!*graph) {
    (void)hipGraphExecDestroy(exec);
    return MOE_ERR_HIP;
  }
  return MOE_OK;
}

MOE_API int moe_graph_launch(moe_graph* graph, void* stream) {
  if (!graph) return MOE_ERR_NULL_PTR;
  if (!graph->exec) return MOE_OK;  // T = 0
  return to_status(hipGraphLaunch(graph->exec, static_cast<hipStream_t>(stream)));
}

MOE_API int moe_graph_destroy(moe_graph* graph) {
  if (!graph) return MOE_OK;
  const hipError_t e = graph->exec ? hipGraphExecDestroy(graph->exec) : hipSuccess;
  delete graph;
  return to_status(e);
}

MOE_API int moe_timing_enable(int kind_mask) {
  if (kind_mask < 0 || kind_mask >= (1 << MOE_KERNEL_COUNT)) return MOE_ERR_BAD_ARG;
  std::lock_guard<std::mutex> lk(g_timing_mu);
  g_timing_mask = static_cast<uint32_t>(kind_mask);
  return MOE_OK;
}

MOE_API int moe_timing_collect(double* total_ms, int64_t* launches, int reset) {
  std::vector<Pending> pend;
  {
    std::lock_guard<std::mutex> lk(g_timing_mu);
    pend.swap(g_pending);
  }
  int status = MOE_OK;
  std::vector<std::pair<int, float>> done;
  for (const Pending& q : pend) {
    float ms = 0.f;
    if (hipEventSynchronize(q.stop) != hipSuccess ||
        hipEventElapsedTime(&ms, q.start, q.stop) != hipSuccess)
      status = MOE_ERR_HIP;
    else
      done.push_back({q.kind, ms});
  }
  std::lock_guard<std::mutex> lk(g_timing_mu);
  for (const Pending& q : pend) g_event_pool.push_back({q.start, q.stop});
  for (const auto& dk : done) {
    g_total_ms[dk.first] += dk.second;
    g_launches[dk.first] += 1;
  }
  for (int i = 0; i < MOE_KERNEL_COUNT; ++i) {
    if (total_ms) total_ms[i] = g_total_ms[i];
    if (launches) launches[i] = g_launches[i];
    if (reset) {
      g_total_ms[i] = 0.0;
      g_launches[i] = 0;
    }
  }
  return status;
}

MOE_API const char* moe_kernel_name(int kind) {
  static const char* names[MOE_KERNEL_COUNT] = {"route_logits", "route_topk", "align",
                                                "ffn13",        "ffn2",       "combine",
                                                "quant_x",      "ffn_fused"};
  return (kind >= 0 && kind < MOE_KERNEL_COUNT) ? names[kind] : "";
}

}  // extern "C"
