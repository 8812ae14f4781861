// beamstep.hip -- host runtime of libbeamstep.so (gfx950), and the one
// translation unit that includes the kernels.
//
// One decode step of batched beam search ("llm_internals" 9.2.2: expand,
// score, prune, finalize; the batched section of "Transformers中的Beam
// Search高效实现") as two kernels plus the KV-cache reorder, and the verify
// step of blockwise parallel decoding ("Blockwise Parallel Decoding",
// section 3):
//
//   K1 expand_select   (select_fused.h) grid (tiles, rows). Streams each live
//                      row's logits once with 16-byte loads. Per (row, tile)
//                      it leaves the online softmax partial (max m, sum
//                      exp(x - m)) and the tile's K best raw logits ordered by
//                      (x desc, v asc). Log-softmax is monotone within a row,
//                      so the union of the tile lists holds the row's best K
//                      candidates.
//   K2 select_finalize (select_fused.h) grid (B). lse per row from the
//                      partials, a K-round merge of the sorted tile lists per
//                      row and then across rows by (cand desc, j asc), then the
//                      finalize sub-step: EOS selections into the finished set
//                      with the length penalty, compaction of live slots in
//                      rank order, backpointers, the stop rule, and the plan
//                      for the KV reorder.
//   K3 kv_reorder      (kv_reorder.h) grid (tiles, B, planes). Each thread
//                      reads one 16-byte word of every distinct parent row,
//                      waits, and writes it to every slot that moved, so swaps
//                      and cycles are safe in place and a shared parent is
//                      read once.
//   K4 verify          (verify.h) argmax and proposal ranks per row, then one
//                      wave per item forms the accepted prefix.
//   K5 finalize        (search_state.h) grid (B). Final ranking and backtrace.
//   L1-L3              (select_two_pass.h) the coarse-to-fine selection of the
//                      LightSeq article ("层级式解码计算"), selectable instead
//                      of K1/K2.
//   K6/K7              (kv_paged.h) the paged KV cache: block tables and the
//                      copies on write.
//
// No matrix cores: nothing here is a dense contraction. Every kernel is bound
// by HBM bandwidth or, at small shapes, by latency.

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>

#include "beamstep.h"

#pragma clang fp contract(off)

#include "device_common.h"
#include "select_fused.h"
#include "select_two_pass.h"
#include "kv_reorder.h"
#include "verify.h"
#include "search_state.h"
#include "kv_paged.h"
#include "init.h"

// ===========================================================================
// host runtime
// ===========================================================================

struct bs_state {
  bs_config cfg;
  hipStream_t stream;
  int device;
  int B, W, V, T, rows, wmax, ept, tile, tiles;
  int K, kmax;          // candidates ranked per item (W or 2W), pow2 bound
  int t;                // steps taken
  void* block;          // the one device allocation
  DevState st;
  double* lpt;
  float* pm;
  float* ps;
  float* px;
  int* pv;
  // two-pass selection
  int KP, cap;
  float* gm;
  float* qc;
  int* qj;
  int* qn;
  bs_kv_paged* paged;   // the paged cache whose table update bs_step runs
  bs_kv_paged* caches;  // every paged cache created on the handle (linked)
};

struct bs_kv_paged {
  bs_state* h;          // null once the handle is destroyed (the cache is orphaned)
  bs_kv_paged* next;    // the handle's next cache
  hipStream_t stream;   // the handle's stream
  int bs, bpi, mb;
  int last_t;   // the step last reordered (0: none since the reset)
  int table_t;  // the step whose table update has run (0: none since the reset)
  void* block;
  PagedDev pg;
};

struct bs_verify_state {
  hipStream_t stream;
  int device;
  int B, k, V, dtype, ept, tile, tiles;
  void* block;
  float* px;
  int* pv;
  int* pc;
};

namespace {

int pow2ceil(int n) {
  int p = 1;
  while (p < n) p <<= 1;
  return p;
}

size_t align_up(size_t n) { return (n + 255) & ~(size_t)255; }

int choose_ept(int rows, int V, int hint) {
  if (hint == 16 || hint == 32 || hint == 64) return hint;
  // 32 logits per thread when that still gives >= 1024 workgroups, else 16.
  // At the wide shape (256 rows, V = 250000) K1 + K2 took 60.6 us per step
  // with 32, 64.8 with 64 and 84 with 16 (62 tiles per row lengthen K2's
  // merge); the Llama-3-8B and Transformer-base shapes get 16 (32 gives 512
  // workgroups there and measured no faster).
  const int64_t tiles32 = (V + (int64_t)kThreads * 32 - 1) / ((int64_t)kThreads * 32);
  return (int64_t)rows * tiles32 >= 1024 ? 32 : 16;
}

int launch_status() { return hipGetLastError() == hipSuccess ? BS_OK : BS_EDEVICE; }

// ---- K1 dispatch ----------------------------------------------------------
template <int WMAX, typename T, int EPT>
void launch_k1_a(const K1Args& a, bool aligned, dim3 grid, hipStream_t s) {
  if (aligned)
    hipLaunchKernelGGL((k1_expand_select<WMAX, T, EPT, true>), grid, dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL((k1_expand_select<WMAX, T, EPT, false>), grid, dim3(kThreads), 0, s, a);
}
template <int WMAX, typename T>
void launch_k1_e(const K1Args& a, int ept, bool aligned, dim3 grid, hipStream_t s) {
  if (ept == 64) launch_k1_a<WMAX, T, 64>(a, aligned, grid, s);
  else if (ept == 32) launch_k1_a<WMAX, T, 32>(a, aligned, grid, s);
  else launch_k1_a<WMAX, T, 16>(a, aligned, grid, s);
}
template <int WMAX>
void launch_k1_t(const K1Args& a, int dtype, int ept, bool aligned, dim3 grid, hipStream_t s) {
  if (dtype == BS_BF16) launch_k1_e<WMAX, uint16_t>(a, ept, aligned, grid, s);
  else launch_k1_e<WMAX, float>(a, ept, aligned, grid, s);
}
void launch_k1(const K1Args& a, int wmax, int dtype, int ept, bool aligned, dim3 grid,
               hipStream_t s) {
  switch (wmax) {
    case 1: launch_k1_t<1>(a, dtype, ept, aligned, grid, s); break;
    case 2: launch_k1_t<2>(a, dtype, ept, aligned, grid, s); break;
    case 4: launch_k1_t<4>(a, dtype, ept, aligned, grid, s); break;
    case 8: launch_k1_t<8>(a, dtype, ept, aligned, grid, s); break;
    default: launch_k1_t<16>(a, dtype, ept, aligned, grid, s); break;
  }
}

template <typename T, int EPT>
void launch_cf_a(const CFArgs& a, bool aligned, dim3 grid, hipStream_t s) {
  if (aligned) {
    hipLaunchKernelGGL((l1_coarse<T, EPT, true>), grid, dim3(kThreads), 0, s, a);
    hipLaunchKernelGGL((l2_fine<T, EPT, true>), grid, dim3(kThreads), 0, s, a);
  } else {
    hipLaunchKernelGGL((l1_coarse<T, EPT, false>), grid, dim3(kThreads), 0, s, a);
    hipLaunchKernelGGL((l2_fine<T, EPT, false>), grid, dim3(kThreads), 0, s, a);
  }
}
template <typename T>
void launch_cf_t(const CFArgs& a, int ept, bool aligned, dim3 grid, hipStream_t s) {
  if (ept == 64) launch_cf_a<T, 64>(a, aligned, grid, s);
  else if (ept == 32) launch_cf_a<T, 32>(a, aligned, grid, s);
  else launch_cf_a<T, 16>(a, aligned, grid, s);
}
template <typename T>
void launch_l3_t(const L3Args& a, int wmax, hipStream_t s) {
  dim3 g(a.k2.B), blk(kThreads);
  switch (wmax) {
    case 1: hipLaunchKernelGGL((l3_sort_finalize<1, T>), g, blk, 0, s, a); break;
    case 2: hipLaunchKernelGGL((l3_sort_finalize<2, T>), g, blk, 0, s, a); break;
    case 4: hipLaunchKernelGGL((l3_sort_finalize<4, T>), g, blk, 0, s, a); break;
    case 8: hipLaunchKernelGGL((l3_sort_finalize<8, T>), g, blk, 0, s, a); break;
    default: hipLaunchKernelGGL((l3_sort_finalize<16, T>), g, blk, 0, s, a); break;
  }
}

// K2 can run the paged cache's table update of the step in the same launch
// (k2_select_finalize_paged) when rows have at most 64 tiles
bool k2_fuses_paged(int tiles) { return tiles <= 64; }

void launch_k2(const K2Args& a, int wmax, hipStream_t s, const K6Args* paged = nullptr) {
  dim3 g(a.B), blk(kThreads);
  // with at most 4 beams the selection's 16-lane row groups fit one wave, so
  // k2_select_finalize runs on 64 threads (measured 0.2% more beam steps/s at
  // the Llama-3-8B shape, 0.6% at Transformer-base); the paged update needs
  // the whole workgroup
  const dim3 blk1(wmax <= 4 && !paged ? 64 : kThreads);
  if (a.tiles <= 64) {
    const int H = a.tiles <= 16 ? 1 : (a.tiles <= 32 ? 2 : 4);  // tiles per lane
    switch (wmax * 8 + H) {
#define K2SEL(WM, HH)                                                                      \
  case WM * 8 + HH:                                                                        \
    if (paged)                                                                             \
      hipLaunchKernelGGL((k2_select_finalize_paged<WM, HH>), g, blk, 0, s, a, *paged);     \
    else                                                                                   \
      hipLaunchKernelGGL((k2_select_finalize<WM, HH>), g, blk1, 0, s, a);                  \
    break;
      K2SEL(1, 1) K2SEL(1, 2) K2SEL(1, 4)
      K2SEL(2, 1) K2SEL(2, 2) K2SEL(2, 4)
      K2SEL(4, 1) K2SEL(4, 2) K2SEL(4, 4)
      K2SEL(8, 1) K2SEL(8, 2) K2SEL(8, 4)
      K2SEL(16, 1) K2SEL(16, 2) K2SEL(16, 4)
#undef K2SEL
      default: break;
    }
    return;
  }
  switch (wmax) {
    case 1: hipLaunchKernelGGL((k2_merge_finalize<1>), g, blk, 0, s, a); break;
    case 2: hipLaunchKernelGGL((k2_merge_finalize<2>), g, blk, 0, s, a); break;
    case 4: hipLaunchKernelGGL((k2_merge_finalize<4>), g, blk, 0, s, a); break;
    case 8: hipLaunchKernelGGL((k2_merge_finalize<8>), g, blk, 0, s, a); break;
    default: hipLaunchKernelGGL((k2_merge_finalize<16>), g, blk, 0, s, a); break;
  }
}

// ---- K3 dispatch ----------------------------------------------------------
// one 16-byte word per thread and parent, one wave per workgroup
// (kK3Threads): more threads with fewer stores in flight each measured faster
// than 2, 4 or 8 words per thread, and smaller workgroups faster than larger
constexpr int kK3Words = 1;
// workgroups along a row: the grid's x extent times the workgroup size must
// stay below 2^32 work-items
constexpr int64_t kK3MaxTiles = 0xFFFFFFFFll / kK3Threads;

// Timing events (either may be null) are attached to the dispatch itself
// (hipExtLaunchKernel), so they take the kernel's own start and end and put
// no separate record on the stream.
struct LaunchEvents {
  hipEvent_t start = nullptr, stop = nullptr;
};

template <int WMAX, int WORD, bool CONTIG>
void launch_k3_c(const K3Args& a, int B, int nplanes, hipStream_t s, LaunchEvents ev) {
  constexpr int NP = kK3Words;
  const int64_t tiles = (a.words + (int64_t)kK3Threads * NP - 1) / ((int64_t)kK3Threads * NP);
  dim3 g((unsigned)tiles, B, nplanes);
  if (ev.start || ev.stop)
    hipExtLaunchKernelGGL((k3_kv_reorder<WMAX, WORD, NP, CONTIG>), g, dim3(kK3Threads), 0, s,
                          ev.start, ev.stop, 0, a);
  else
    hipLaunchKernelGGL((k3_kv_reorder<WMAX, WORD, NP, CONTIG>), g, dim3(kK3Threads), 0, s, a);
}
template <int WMAX>
void launch_k3_w(const K3Args& a, int word, bool contig, int B, int nplanes, hipStream_t s,
                 LaunchEvents ev) {
  if (word == 16) {
    if (contig) launch_k3_c<WMAX, 16, true>(a, B, nplanes, s, ev);
    else launch_k3_c<WMAX, 16, false>(a, B, nplanes, s, ev);
  } else {
    if (contig) launch_k3_c<WMAX, 4, true>(a, B, nplanes, s, ev);
    else launch_k3_c<WMAX, 4, false>(a, B, nplanes, s, ev);
  }
}
void launch_k3(const K3Args& a, int wmax, int word, bool contig, int B, int nplanes,
               hipStream_t s, LaunchEvents ev) {
  switch (wmax) {
    case 1: launch_k3_w<1>(a, word, contig, B, nplanes, s, ev); break;
    case 2: launch_k3_w<2>(a, word, contig, B, nplanes, s, ev); break;
    case 4: launch_k3_w<4>(a, word, contig, B, nplanes, s, ev); break;
    case 8: launch_k3_w<8>(a, word, contig, B, nplanes, s, ev); break;
    default: launch_k3_w<16>(a, word, contig, B, nplanes, s, ev); break;
  }
}

void launch_k5(const K5Args& a, int wmax, hipStream_t s) {
  dim3 g(a.B), blk(64);
  switch (wmax) {
    case 1: hipLaunchKernelGGL((k5_finalize<1>), g, blk, 0, s, a); break;
    case 2: hipLaunchKernelGGL((k5_finalize<2>), g, blk, 0, s, a); break;
    case 4: hipLaunchKernelGGL((k5_finalize<4>), g, blk, 0, s, a); break;
    case 8: hipLaunchKernelGGL((k5_finalize<8>), g, blk, 0, s, a); break;
    default: hipLaunchKernelGGL((k5_finalize<16>), g, blk, 0, s, a); break;
  }
}

// ---- K4 dispatch ----------------------------------------------------------
template <typename T, int EPT, bool COUNT>
void launch_k4_a(const K4Args& a, bool aligned, dim3 grid, hipStream_t s) {
  if (aligned)
    hipLaunchKernelGGL((k4_verify<T, EPT, true, COUNT>), grid, dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL((k4_verify<T, EPT, false, COUNT>), grid, dim3(kThreads), 0, s, a);
}

void fill_k2_args(K2Args& a2, bs_state* h, int t, int32_t* beam_idx, int32_t* token_id,
                  float* scores, uint8_t* done) {
  a2.st = h->st;
  a2.pm = h->pm;
  a2.ps = h->ps;
  a2.px = h->px;
  a2.pv = h->pv;
  a2.B = h->B;
  a2.W = h->W;
  a2.K = h->K;
  a2.V = h->V;
  a2.T = h->T;
  a2.tiles = h->tiles;
  a2.eos = h->cfg.eos_id;
  a2.pad = h->cfg.pad_id;
  a2.stop = h->cfg.stop;
  a2.alpha = h->cfg.alpha;
  a2.t = t;
  a2.out_beam = beam_idx;
  a2.out_tok = token_id;
  a2.out_score = scores;
  a2.out_done = done;
}

void fill_k6_args(K6Args& a6, const bs_kv_paged* p, const bs_state* h, int t) {
  a6.pg = p->pg;
  a6.s = h->st.s;
  a6.done = h->st.done;
  a6.plan = h->st.plan;
  a6.W = h->W;
  a6.bs = p->bs;
  a6.bpi = p->bpi;
  a6.mb = p->mb;
  a6.t = t;
}

constexpr int kRowVerifyMinRows = 256;
constexpr int kVerifySegWorkgroups = 1024;
// row segments of the verify row kernel: enough workgroups to keep every CU
// streaming, never more than the tiles the partials hold
int verify_segments(int rows, int tiles) {
  const int want = (kVerifySegWorkgroups + rows - 1) / rows;
  return want < 1 ? 1 : (want > tiles ? tiles : want);
}

template <typename T, bool COUNT>
void launch_k4_row(const K4Args& a, bool aligned, int rows, hipStream_t s) {
  const dim3 grid(a.tiles, rows);  // segments x rows
  if (aligned)
    hipLaunchKernelGGL((k4_row<T, true, COUNT>), grid, dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL((k4_row<T, false, COUNT>), grid, dim3(kThreads), 0, s, a);
}

void launch_k4_tiles(const K4Args& a, int dtype, bool count, bool aligned, dim3 grid,
                     hipStream_t s) {
  if (count) {
    if (dtype == BS_BF16) launch_k4_a<uint16_t, 16, true>(a, aligned, grid, s);
    else launch_k4_a<float, 16, true>(a, aligned, grid, s);
  } else {
    if (dtype == BS_BF16) launch_k4_a<uint16_t, 16, false>(a, aligned, grid, s);
    else launch_k4_a<float, 16, false>(a, aligned, grid, s);
  }
}

// The verify call's launches: the row or tile kernel writes one partial
// (maximum, its first column, and with COUNT the logits that beat the
// proposal's) per (row, segment or tile) into px/pv/pc, then k4_accept merges
// them; every partial is written before it is read, so the buffers need no
// clearing. tiles: the logits' tiles of kThreads * 16 elements per row.
int verify_segments_for(int rows, int tiles) {
  return rows >= kRowVerifyMinRows ? verify_segments(rows, tiles) : tiles;
}

int launch_verify(hipStream_t s, int dtype, int B, int k, int V, int tiles, const void* logits,
                  int64_t stride, const int32_t* proposals, int top_k, int min_block,
                  int32_t* accept_len, int32_t* argmax, int32_t* prop_rank, float* px, int* pv,
                  int* pc) {
  const int esize = dtype == BS_BF16 ? 2 : 4;
  const bool aligned = ((uintptr_t)logits % 16 == 0) && ((stride * esize) % 16 == 0);
  const bool count = top_k > 1 || prop_rank != nullptr;
  K4Args a;
  a.logits = logits;
  a.stride = stride;
  a.V = V;
  a.tile = kThreads * 16;
  a.tiles = tiles;
  a.k = k;
  a.B = B;
  a.px = px;
  a.pv = pv;
  a.pc = pc;
  a.proposals = proposals;
  a.accept = accept_len;
  a.argmax = argmax;
  a.rank = prop_rank;
  a.top_k = top_k;
  a.min_block = min_block;
  const int rows = B * k;
  if (rows >= kRowVerifyMinRows) {
    // enough rows to fill the chip: a few segments per row, one tile each
    a.tiles = verify_segments(rows, tiles);
    if (dtype == BS_BF16) {
      if (count) launch_k4_row<uint16_t, true>(a, aligned, rows, s);
      else launch_k4_row<uint16_t, false>(a, aligned, rows, s);
    } else {
      if (count) launch_k4_row<float, true>(a, aligned, rows, s);
      else launch_k4_row<float, false>(a, aligned, rows, s);
    }
  } else {
    launch_k4_tiles(a, dtype, count, aligned, dim3(tiles, rows), s);
  }
  int rc = launch_status();
  if (rc != BS_OK) return rc;
  if (count)
    hipLaunchKernelGGL((k4_accept<true>), dim3(B), dim3(64), 0, s, a);
  else
    hipLaunchKernelGGL((k4_accept<false>), dim3(B), dim3(64), 0, s, a);
  return launch_status();
}

int launch_init(bs_state* h) {
  InitArgs ia;
  ia.st = h->st;
  ia.lpt = h->lpt;
  ia.qn = h->qn;
  ia.B = h->B;
  ia.W = h->W;
  ia.T = h->T;
  ia.lp = h->cfg.lp;
  ia.alpha = h->cfg.alpha;
  int n = h->B * h->W;
  if (h->T + 1 > n) n = h->T + 1;
  hipLaunchKernelGGL(k0_init, dim3((n + 255) / 256), dim3(256), 0, h->stream, ia);
  return launch_status();
}

}  // namespace

// ---- workspace of bs_verify_noalloc ---------------------------------------
// For callers that cannot allocate device memory, the verify call's partials
// live in this array instead of a handle's allocation: each GPU the library
// runs on holds its own copy until the process ends, and every
// bs_verify_noalloc call on that GPU uses it (calls that overlap on one GPU
// race). Host code never passes `scratch` itself to a kernel -- in host code
// the name is a host-side stand-in -- but the device address that
// hipGetSymbolAddress gives for the current device, looked up once per device.
constexpr size_t kScratchBytes = (size_t)4 << 20;
static __device__ __align__(256) char scratch[kScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// the current device's address of `scratch`
int scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return BS_EDEVICE;
  if (dev < 0 || dev >= kMaxDevices) return BS_EDEVICE;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      (void)hipGetLastError();
      return BS_EDEVICE;
    }
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return BS_OK;
}
}  // namespace

extern "C" {

const char* bs_strerror(int status) {
  switch (status) {
    case BS_OK: return "ok";
    case BS_EINVAL: return "invalid argument";
    case BS_ENOMEM: return "device allocation failed";
    case BS_EDEVICE: return "HIP runtime error";
    case BS_ESTATE: return "call not valid in the current state";
    default: return "unknown status";
  }
}

int bs_create(const bs_config* cfg, void* hip_stream, bs_state** out) {
  if (!cfg || !out) return BS_EINVAL;
  *out = nullptr;
  const bs_config c = *cfg;
  if (c.batch < 1 || c.beam < 1 || c.beam > kMaxBeam || c.vocab < 1 || c.max_steps < 1)
    return BS_EINVAL;
  if ((int64_t)c.beam * c.vocab >= ((int64_t)1 << 31)) return BS_EINVAL;
  if ((int64_t)c.batch * c.beam > kMaxGridRows) return BS_EINVAL;
  if ((int64_t)c.batch * c.beam * c.max_steps >= ((int64_t)1 << 31)) return BS_EINVAL;
  if (c.logits_dtype != BS_F32 && c.logits_dtype != BS_BF16) return BS_EINVAL;
  if (c.lp < BS_LP_NONE || c.lp > BS_LP_POW) return BS_EINVAL;
  if (c.stop < BS_STOP_TRUE || c.stop > BS_STOP_NEVER) return BS_EINVAL;
  if (c.num_return < 1 || c.num_return > c.beam) return BS_EINVAL;
  if (c.tile_elems != 0 && c.tile_elems != 16 && c.tile_elems != 32 && c.tile_elems != 64)
    return BS_EINVAL;
  if (!isfinite(c.alpha)) return BS_EINVAL;
  if (c.prune != BS_PRUNE_TOPW && c.prune != BS_PRUNE_TOP2W) return BS_EINVAL;
  if (c.prune == BS_PRUNE_TOP2W && 2 * c.beam > kMaxBeam) return BS_EINVAL;
  if (c.select != BS_SELECT_FUSED && c.select != BS_SELECT_TWO_PASS) return BS_EINVAL;

  bs_state* h = (bs_state*)calloc(1, sizeof(bs_state));
  if (!h) return BS_ENOMEM;
  h->cfg = c;
  h->stream = (hipStream_t)hip_stream;
  if (hipGetDevice(&h->device) != hipSuccess) {
    free(h);
    return BS_EDEVICE;
  }
  h->B = c.batch;
  h->W = c.beam;
  h->V = c.vocab;
  h->T = c.max_steps;
  h->rows = c.batch * c.beam;
  h->wmax = pow2ceil(c.beam);
  h->K = c.prune == BS_PRUNE_TOP2W ? 2 * c.beam : c.beam;
  h->kmax = pow2ceil(h->K);
  h->ept = choose_ept(h->rows, c.vocab, c.tile_elems);
  h->tile = kThreads * h->ept;
  h->tiles = (c.vocab + h->tile - 1) / h->tile;

  const size_t RW = (size_t)h->rows;
  const size_t PT = RW * h->tiles;
  const size_t BT = (size_t)h->T * RW;
  const bool two = c.select == BS_SELECT_TWO_PASS;
  h->KP = pow2ceil(h->K);
  h->cap = kThreads * h->KP;
  size_t sizes[] = {
      RW * 4,                 // s
      RW * 4,                 // slot_rank
      (size_t)h->B,           // done
      RW * 4, RW * 4, RW * 4, RW * 4, RW * 4, RW * 4, RW * 4,  // finished set
      (size_t)h->B * 4,       // hcount
      BT * 4, BT * 4,         // backpointers
      (size_t)h->B * h->K * 4, (size_t)h->B * h->K * 4,  // selection
      (size_t)h->B * kPlanStride * 4,  // plan
      ((size_t)h->T + 1) * 8, // lpt
      PT * 4, PT * 4,         // pm, ps
      PT * h->kmax * 4, PT * h->kmax * 4,  // px, pv
      two ? PT * h->KP * 4 : 0,            // two-pass: group maxima
      two ? (size_t)h->B * h->cap * 4 : 0, two ? (size_t)h->B * h->cap * 4 : 0,  // queue
      two ? (size_t)h->B * 4 : 0,          // queue lengths
  };
  const int n = sizeof(sizes) / sizeof(sizes[0]);
  size_t total = 0;
  for (int i = 0; i < n; ++i) total += align_up(sizes[i]);
  if (hipMalloc(&h->block, total) != hipSuccess) {
    (void)hipGetLastError();
    free(h);
    return BS_ENOMEM;
  }
  char* p = (char*)h->block;
  void* ptr[n];
  for (int i = 0; i < n; ++i) {
    ptr[i] = p;
    p += align_up(sizes[i]);
  }
  int i = 0;
  h->st.s = (float*)ptr[i++];
  h->st.slot_rank = (int*)ptr[i++];
  h->st.done = (uint8_t*)ptr[i++];
  h->st.hnorm = (float*)ptr[i++];
  h->st.hraw = (float*)ptr[i++];
  h->st.hlen = (int*)ptr[i++];
  h->st.hstep = (int*)ptr[i++];
  h->st.hrank = (int*)ptr[i++];
  h->st.hpar = (int*)ptr[i++];
  h->st.htok = (int*)ptr[i++];
  h->st.hcount = (int*)ptr[i++];
  h->st.bp_par = (int*)ptr[i++];
  h->st.bp_tok = (int*)ptr[i++];
  h->st.sel_j = (int*)ptr[i++];
  h->st.sel_c = (float*)ptr[i++];
  h->st.plan = (int*)ptr[i++];
  h->lpt = (double*)ptr[i++];
  h->st.lpt = h->lpt;
  h->pm = (float*)ptr[i++];
  h->ps = (float*)ptr[i++];
  h->px = (float*)ptr[i++];
  h->pv = (int*)ptr[i++];
  h->gm = two ? (float*)ptr[i] : nullptr;
  ++i;
  h->qc = two ? (float*)ptr[i] : nullptr;
  ++i;
  h->qj = two ? (int*)ptr[i] : nullptr;
  ++i;
  h->qn = two ? (int*)ptr[i] : nullptr;
  ++i;

  int rc = launch_init(h);
  if (rc == BS_OK && hipStreamSynchronize(h->stream) != hipSuccess) rc = BS_EDEVICE;
  if (rc != BS_OK) {
    (void)hipFree(h->block);
    free(h);
    return rc;
  }
  *out = h;
  return BS_OK;
}

int bs_reset(bs_state* h) {
  if (!h) return BS_EINVAL;
  int rc = launch_init(h);
  if (rc == BS_OK) h->t = 0;
  return rc;
}

int bs_step(bs_state* h, const void* logits, int64_t row_stride_elems, int32_t* beam_idx,
            int32_t* token_id, float* scores, uint8_t* done) {
  if (!h || !logits || !beam_idx || !token_id || !scores || !done) return BS_EINVAL;
  if (row_stride_elems < h->V) return BS_EINVAL;
  if (h->t >= h->T) return BS_ESTATE;
  const int t = h->t + 1;
  const int esize = h->cfg.logits_dtype == BS_BF16 ? 2 : 4;
  const bool aligned = ((uintptr_t)logits % 16 == 0) && ((row_stride_elems * esize) % 16 == 0);

  if (h->cfg.select == BS_SELECT_TWO_PASS) {
    CFArgs cf;
    cf.logits = logits;
    cf.stride = row_stride_elems;
    cf.V = h->V;
    cf.W = h->W;
    cf.K = h->K;
    cf.KP = h->KP;
    cf.tile = h->tile;
    cf.tiles = h->tiles;
    cf.s = h->st.s;
    cf.done = h->st.done;
    cf.pm = h->pm;
    cf.ps = h->ps;
    cf.gm = h->gm;
    cf.qc = h->qc;
    cf.qj = h->qj;
    cf.qn = h->qn;
    cf.cap = h->cap;
    const dim3 grid(h->tiles, h->rows);
    if (h->cfg.logits_dtype == BS_BF16) launch_cf_t<uint16_t>(cf, h->ept, aligned, grid, h->stream);
    else launch_cf_t<float>(cf, h->ept, aligned, grid, h->stream);
    int rc = launch_status();
    if (rc != BS_OK) return rc;
    L3Args a3;
    a3.cf = cf;
    fill_k2_args(a3.k2, h, t, beam_idx, token_id, scores, done);
    if (h->cfg.logits_dtype == BS_BF16) launch_l3_t<uint16_t>(a3, h->kmax, h->stream);
    else launch_l3_t<float>(a3, h->kmax, h->stream);
    rc = launch_status();
    if (rc != BS_OK) return rc;
    h->t = t;
    return BS_OK;
  }

  K1Args a1;
  a1.logits = logits;
  a1.stride = row_stride_elems;
  a1.V = h->V;
  a1.W = h->W;
  a1.K = h->K;
  a1.tile = h->tile;
  a1.tiles = h->tiles;
  a1.s = h->st.s;
  a1.done = h->st.done;
  a1.pm = h->pm;
  a1.ps = h->ps;
  a1.px = h->px;
  a1.pv = h->pv;
  launch_k1(a1, h->kmax, h->cfg.logits_dtype, h->ept, aligned, dim3(h->tiles, h->rows),
            h->stream);
  int rc = launch_status();
  if (rc != BS_OK) return rc;

  K2Args a2;
  fill_k2_args(a2, h, t, beam_idx, token_id, scores, done);
  // the handle's paged cache, when every earlier step of the search has been
  // reordered: K2 also runs this step's table update, and the reorder call
  // only copies
  bs_kv_paged* p = h->paged;
  const bool fuse = p && k2_fuses_paged(h->tiles) && p->last_t == h->t && p->table_t == h->t;
  K6Args a6;
  if (fuse) fill_k6_args(a6, p, h, t);
  launch_k2(a2, h->kmax, h->stream, fuse ? &a6 : nullptr);
  rc = launch_status();
  if (rc != BS_OK) return rc;
  if (fuse) p->table_t = t;
  h->t = t;
  return BS_OK;
}

// n * stride + bytes <= limit, without overflow (all >= 0)
static bool span_within(int64_t n, int64_t stride, int64_t bytes, int64_t limit) {
  if (bytes > limit) return false;
  return n == 0 || stride <= (limit - bytes) / n;
}

static int reorder_kv(bs_state* h, const bs_kv_desc* kv, int32_t gen_len, LaunchEvents ev) {
  if (!h || !kv || !kv->planes || kv->n_planes < 1 || gen_len < 0) return BS_EINVAL;
  if (kv->bytes_per_pos <= 0 || kv->row_stride <= 0 || kv->pos_stride <= 0 || kv->pos_offset < 0)
    return BS_EINVAL;
  // the moved (row, position) pairs of a plane must not share bytes: positions
  // apart within a row, and either rows apart by the moved span of a row
  // (row-major) or positions apart by every row (position-major)
  const int64_t rows = (int64_t)h->B * h->W;
  const bool row_major = span_within(gen_len > 0 ? gen_len - 1 : 0, kv->pos_stride,
                                     kv->bytes_per_pos, kv->row_stride);
  const bool pos_major = kv->bytes_per_pos <= kv->row_stride &&
                         span_within(rows - 1, kv->row_stride, kv->bytes_per_pos, kv->pos_stride);
  if (kv->bytes_per_pos > kv->pos_stride || !(row_major || pos_major)) return BS_EINVAL;
  if (h->t == 0) return BS_ESTATE;
  if (gen_len == 0) {  // nothing to launch: the events are recorded back to back
    if ((ev.start && hipEventRecord(ev.start, h->stream) != hipSuccess) ||
        (ev.stop && hipEventRecord(ev.stop, h->stream) != hipSuccess))
      return BS_EDEVICE;
    return BS_OK;
  }
  const int64_t base_off = kv->pos_offset * kv->pos_stride;
  bool a16 = (kv->bytes_per_pos % 16 == 0) && (kv->row_stride % 16 == 0) &&
             (kv->pos_stride % 16 == 0) && (base_off % 16 == 0);
  bool a4 = (kv->bytes_per_pos % 4 == 0) && (kv->row_stride % 4 == 0) &&
            (kv->pos_stride % 4 == 0) && (base_off % 4 == 0);
  for (int i = 0; i < kv->n_planes; ++i) {
    if (!kv->planes[i]) return BS_EINVAL;
    a16 = a16 && ((uintptr_t)kv->planes[i] % 16 == 0);
    a4 = a4 && ((uintptr_t)kv->planes[i] % 4 == 0);
  }
  if (!a4) return BS_EINVAL;
  const int word = a16 ? 16 : 4;
  const bool contig = kv->pos_stride == kv->bytes_per_pos;
  K3Args a;
  a.row_stride = kv->row_stride;
  a.pos_stride = kv->pos_stride;
  a.base_off = base_off;
  a.words_per_pos = kv->bytes_per_pos / word;
  a.words = (int64_t)gen_len * a.words_per_pos;
  if ((a.words + kK3Threads * kK3Words - 1) / (kK3Threads * kK3Words) > kK3MaxTiles)
    return BS_EINVAL;
  a.W = h->W;
  a.plan = h->st.plan;
  for (int p0 = 0; p0 < kv->n_planes; p0 += kMaxPlanesPerLaunch) {
    const int np = kv->n_planes - p0 < kMaxPlanesPerLaunch ? kv->n_planes - p0
                                                           : kMaxPlanesPerLaunch;
    for (int i = 0; i < np; ++i) a.planes[i] = (char*)kv->planes[p0 + i];
    // the start event goes with the first launch of the call, the stop event
    // with the last
    LaunchEvents le;
    le.start = p0 == 0 ? ev.start : nullptr;
    le.stop = p0 + np == kv->n_planes ? ev.stop : nullptr;
    launch_k3(a, h->wmax, word, contig, h->B, np, h->stream, le);
    const int rc = launch_status();
    if (rc != BS_OK) return rc;
  }
  return BS_OK;
}

int bs_reorder_kv(bs_state* h, const bs_kv_desc* kv, int32_t gen_len) {
  return reorder_kv(h, kv, gen_len, LaunchEvents());
}

int bs_reorder_kv_timed(bs_state* h, const bs_kv_desc* kv, int32_t gen_len, void* start_event,
                        void* stop_event) {
  LaunchEvents ev;
  ev.start = (hipEvent_t)start_event;
  ev.stop = (hipEvent_t)stop_event;
  return reorder_kv(h, kv, gen_len, ev);
}

int bs_kv_paged_create(bs_state* h, int32_t block_size, int32_t blocks_per_item,
                       bs_kv_paged** out) {
  if (!h || !out) return BS_EINVAL;
  *out = nullptr;
  if (block_size < 1 || blocks_per_item < h->W || blocks_per_item > kPagedMaxBlocks)
    return BS_EINVAL;
  const int mb = h->T / block_size + 1;
  if ((int64_t)h->W * mb > kPagedMaxTable) return BS_EINVAL;
  if ((int64_t)h->B * blocks_per_item >= ((int64_t)1 << 31)) return BS_EINVAL;
  bs_kv_paged* p = (bs_kv_paged*)calloc(1, sizeof(bs_kv_paged));
  if (!p) return BS_ENOMEM;
  p->h = h;
  p->stream = h->stream;
  p->bs = block_size;
  p->bpi = blocks_per_item;
  p->mb = mb;
  const size_t B = (size_t)h->B;
  const size_t sizes[] = {
      B * h->W * mb * 4,            // table
      B * blocks_per_item * 4,      // reference counts
      B * blocks_per_item * 4,      // free lists
      B * 4,                        // free counts
      4,                            // overflow flag
      B * h->W * 3 * 4,             // the step's copy list
      2 * 4,                        // its length, by step parity
  };
  const int n = sizeof(sizes) / sizeof(sizes[0]);
  size_t total = 0;
  for (int i = 0; i < n; ++i) total += align_up(sizes[i]);
  if (hipMalloc(&p->block, total) != hipSuccess) {
    (void)hipGetLastError();
    free(p);
    return BS_ENOMEM;
  }
  char* q = (char*)p->block;
  int* ptr[n];
  for (int i = 0; i < n; ++i) {
    ptr[i] = (int*)q;
    q += align_up(sizes[i]);
  }
  p->pg.table = ptr[0];
  p->pg.refc = ptr[1];
  p->pg.freel = ptr[2];
  p->pg.nfree = ptr[3];
  p->pg.overflow = ptr[4];
  p->pg.cpy = ptr[5];
  p->pg.ncpy = ptr[6];
  int rc = bs_kv_paged_reset(p);
  if (rc == BS_OK && hipStreamSynchronize(h->stream) != hipSuccess) rc = BS_EDEVICE;
  if (rc != BS_OK) {
    (void)hipFree(p->block);
    free(p);
    return rc;
  }
  if (!h->paged) h->paged = p;  // the first cache of a handle: bs_step runs its table update
  p->next = h->caches;
  h->caches = p;
  *out = p;
  return BS_OK;
}

int bs_kv_paged_reset(bs_kv_paged* p) {
  if (!p) return BS_EINVAL;
  if (!p->h) return BS_ESTATE;
  hipLaunchKernelGGL(k6_paged_init, dim3(p->h->B), dim3(kThreads), 0, p->h->stream, p->pg,
                     p->h->B, p->h->W, p->bpi, p->mb);
  const int rc = launch_status();
  if (rc == BS_OK) p->last_t = p->table_t = 0;
  return rc;
}

int bs_kv_paged_table(const bs_kv_paged* p, int32_t** table, int32_t* max_blocks) {
  if (!p || !table || !max_blocks) return BS_EINVAL;
  if (!p->h) return BS_ESTATE;
  *table = p->pg.table;
  *max_blocks = p->mb;
  return BS_OK;
}

int bs_kv_paged_reorder(bs_kv_paged* p, const bs_kv_pool* pool, int32_t gen_len) {
  if (!p || !pool || !pool->pools || pool->n_planes < 1) return BS_EINVAL;
  if (pool->block_stride <= 0 || pool->pos_stride <= 0 || pool->bytes_per_pos <= 0)
    return BS_EINVAL;
  if (pool->bytes_per_pos > pool->pos_stride ||
      (int64_t)(p->bs - 1) * pool->pos_stride + pool->bytes_per_pos > pool->block_stride)
    return BS_EINVAL;
  bs_state* h = p->h;
  if (!h) return BS_ESTATE;
  // every step is reordered once, in order: the table of step t is built on
  // that of step t-1
  if (h->t == 0 || gen_len != h->t || p->last_t + 1 != h->t) return BS_ESTATE;
  bool a16 = (pool->bytes_per_pos % 16 == 0) && (pool->pos_stride % 16 == 0) &&
             (pool->block_stride % 16 == 0);
  bool a4 = (pool->bytes_per_pos % 4 == 0) && (pool->pos_stride % 4 == 0) &&
            (pool->block_stride % 4 == 0);
  for (int i = 0; i < pool->n_planes; ++i) {
    if (!pool->pools[i]) return BS_EINVAL;
    a16 = a16 && ((uintptr_t)pool->pools[i] % 16 == 0);
    a4 = a4 && ((uintptr_t)pool->pools[i] % 4 == 0);
  }
  if (!a4) return BS_EINVAL;
  int rc = BS_OK;
  if (p->table_t != h->t) {  // bs_step did not run the table update of this step
    K6Args a6;
    fill_k6_args(a6, p, h, gen_len);
    hipLaunchKernelGGL(k6_paged_reorder, dim3(h->B), dim3(kThreads), 0, h->stream, a6);
    rc = launch_status();
    if (rc != BS_OK) return rc;
    p->table_t = h->t;
  }
  const int word = a16 ? 16 : 4;
  K7Args a7;
  a7.block_stride = pool->block_stride;
  a7.pos_stride = pool->pos_stride;
  a7.words_per_pos = (int)(pool->bytes_per_pos / word);
  a7.cpy = p->pg.cpy;
  a7.ncpy = p->pg.ncpy;
  a7.parity = gen_len & 1;
  a7.max_copies = h->B * h->W;
  const int64_t words = (int64_t)(p->bs - 1) * a7.words_per_pos;  // at most bs-1 positions
  a7.tiles = (int)((words + kK7Threads - 1) / kK7Threads);
  if (a7.tiles > 0) {
    for (int p0 = 0; p0 < pool->n_planes; p0 += kMaxPlanesPerLaunch) {
      const int np = pool->n_planes - p0 < kMaxPlanesPerLaunch ? pool->n_planes - p0
                                                                : kMaxPlanesPerLaunch;
      a7.n_planes = np;
      a7.groups = (np + kCopyPlanes - 1) / kCopyPlanes;
      for (int i = 0; i < np; ++i) a7.pools[i] = (char*)pool->pools[p0 + i];
      if (word == 16)
        hipLaunchKernelGGL(k7_paged_copy<16>, dim3(kCopyGrid), dim3(kK7Threads), 0, h->stream, a7);
      else
        hipLaunchKernelGGL(k7_paged_copy<4>, dim3(kCopyGrid), dim3(kK7Threads), 0, h->stream, a7);
      rc = launch_status();
      if (rc != BS_OK) return rc;
    }
  }
  p->last_t = h->t;
  return BS_OK;
}

int bs_kv_paged_status(bs_kv_paged* p, int32_t* overflow, int32_t* free_blocks) {
  if (!p || !overflow) return BS_EINVAL;
  if (!p->h) return BS_ESTATE;
  hipStream_t s = p->h->stream;
  if (hipStreamSynchronize(s) != hipSuccess) return BS_EDEVICE;
  if (hipMemcpy(overflow, p->pg.overflow, 4, hipMemcpyDeviceToHost) != hipSuccess)
    return BS_EDEVICE;
  if (free_blocks &&
      hipMemcpy(free_blocks, p->pg.nfree, (size_t)p->h->B * 4, hipMemcpyDeviceToHost) !=
          hipSuccess)
    return BS_EDEVICE;
  return BS_OK;
}

void bs_kv_paged_destroy(bs_kv_paged* p) {
  if (!p) return;
  if (p->h) {  // unlink from the handle
    if (p->h->paged == p) p->h->paged = nullptr;
    for (bs_kv_paged** q = &p->h->caches; *q; q = &(*q)->next)
      if (*q == p) {
        *q = p->next;
        break;
      }
  }
  (void)hipStreamSynchronize(p->stream);
  (void)hipFree(p->block);
  free(p);
}

int bs_finalize(bs_state* h, int32_t* tokens, int32_t* lengths, float* norm_scores) {
  if (!h || !tokens || !lengths || !norm_scores) return BS_EINVAL;
  if (h->t == 0) return BS_ESTATE;
  K5Args a;
  a.st = h->st;
  a.B = h->B;
  a.W = h->W;
  a.T = h->T;
  a.pad = h->cfg.pad_id;
  a.R = h->cfg.num_return;
  a.steps = h->t;
  a.tokens = tokens;
  a.lengths = lengths;
  a.norms = norm_scores;
  launch_k5(a, h->wmax, h->stream);
  return launch_status();
}

int bs_last_selection(bs_state* h, int32_t* flat_idx, float* cand_score) {
  if (!h || !flat_idx || !cand_score) return BS_EINVAL;
  if (h->t == 0) return BS_ESTATE;
  const size_t n = (size_t)h->B * h->K;
  if (hipMemcpyAsync(flat_idx, h->st.sel_j, n * 4, hipMemcpyDeviceToDevice, h->stream) !=
          hipSuccess ||
      hipMemcpyAsync(cand_score, h->st.sel_c, n * 4, hipMemcpyDeviceToDevice, h->stream) !=
          hipSuccess)
    return BS_EDEVICE;
  return BS_OK;
}

int bs_get_finished(bs_state* h, float* norm, float* raw, int32_t* len, int32_t* step,
                    int32_t* rank, int32_t* count) {
  if (!h || !norm || !raw || !len || !step || !rank || !count) return BS_EINVAL;
  const size_t n = (size_t)h->rows * 4;
  const hipMemcpyKind k = hipMemcpyDeviceToDevice;
  if (hipMemcpyAsync(norm, h->st.hnorm, n, k, h->stream) != hipSuccess ||
      hipMemcpyAsync(raw, h->st.hraw, n, k, h->stream) != hipSuccess ||
      hipMemcpyAsync(len, h->st.hlen, n, k, h->stream) != hipSuccess ||
      hipMemcpyAsync(step, h->st.hstep, n, k, h->stream) != hipSuccess ||
      hipMemcpyAsync(rank, h->st.hrank, n, k, h->stream) != hipSuccess ||
      hipMemcpyAsync(count, h->st.hcount, (size_t)h->B * 4, k, h->stream) != hipSuccess)
    return BS_EDEVICE;
  return BS_OK;
}

int bs_steps_taken(const bs_state* h) { return h ? h->t : BS_EINVAL; }

// ---- checkpoint / resume ----------------------------------------------------
// A snapshot is a header (the configuration it belongs to and the steps taken)
// followed by the handle's search state, which bs_create laid out as one
// contiguous range at the start of its allocation: running scores, slot ranks,
// done flags, finished sets, backpointers, the last selection and the reorder
// plan (values only, no addresses). What follows that range (the length-penalty
// table, the per-tile partials) is derived from the configuration or rewritten
// by every step.
namespace {
constexpr uint32_t kSnapMagic = 0x42535331u;  // "BSS1"
struct SnapHeader {
  uint32_t magic, header_bytes;
  int32_t batch, beam, vocab, max_steps, eos_id, pad_id, logits_dtype, lp, stop, num_return;
  int32_t prune, select, steps_taken, reserved;
  double alpha;
  uint64_t state_bytes;
};
static size_t state_bytes(const bs_state* h) { return (size_t)((const char*)h->lpt - (const char*)h->block); }
static SnapHeader snap_header(const bs_state* h) {
  SnapHeader x;
  memset(&x, 0, sizeof(x));
  x.magic = kSnapMagic;
  x.header_bytes = sizeof(SnapHeader);
  x.batch = h->cfg.batch;
  x.beam = h->cfg.beam;
  x.vocab = h->cfg.vocab;
  x.max_steps = h->cfg.max_steps;
  x.eos_id = h->cfg.eos_id;
  x.pad_id = h->cfg.pad_id;
  x.logits_dtype = h->cfg.logits_dtype;
  x.lp = h->cfg.lp;
  x.stop = h->cfg.stop;
  x.num_return = h->cfg.num_return;
  x.prune = h->cfg.prune;
  x.select = h->cfg.select;
  x.steps_taken = h->t;
  x.alpha = h->cfg.alpha;
  x.state_bytes = state_bytes(h);
  return x;
}
}  // namespace

int bs_state_size(const bs_state* h, int64_t* bytes) {
  if (!h || !bytes) return BS_EINVAL;
  *bytes = (int64_t)(sizeof(SnapHeader) + state_bytes(h));
  return BS_OK;
}

int bs_state_save(bs_state* h, void* dst, int64_t capacity) {
  if (!h || !dst) return BS_EINVAL;
  const size_t n = state_bytes(h);
  if (capacity < (int64_t)(sizeof(SnapHeader) + n)) return BS_EINVAL;
  if (hipStreamSynchronize(h->stream) != hipSuccess) return BS_EDEVICE;
  const SnapHeader x = snap_header(h);
  if (hipMemcpy((char*)dst + sizeof(SnapHeader), h->block, n, hipMemcpyDeviceToHost) != hipSuccess)
    return BS_EDEVICE;
  memcpy(dst, &x, sizeof(x));
  return BS_OK;
}

int bs_state_load(bs_state* h, const void* src, int64_t size) {
  if (!h || !src || size < (int64_t)sizeof(SnapHeader)) return BS_EINVAL;
  SnapHeader x, want = snap_header(h);
  memcpy(&x, src, sizeof(x));
  // everything but the step count must be this handle's
  want.steps_taken = x.steps_taken;
  if (memcmp(&x, &want, sizeof(x)) != 0) return BS_EINVAL;
  if (x.steps_taken < 0 || x.steps_taken > h->T) return BS_EINVAL;
  if (size < (int64_t)(sizeof(SnapHeader) + x.state_bytes)) return BS_EINVAL;
  if (hipMemcpyAsync(h->block, (const char*)src + sizeof(SnapHeader), x.state_bytes,
                     hipMemcpyHostToDevice, h->stream) != hipSuccess ||
      hipStreamSynchronize(h->stream) != hipSuccess)
    return BS_EDEVICE;
  h->t = x.steps_taken;
  // the tables of a paged cache belong to the search before the load: the
  // step counts that no step can reach make bs_step leave them alone and their
  // reorders fail with BS_ESTATE until bs_kv_paged_reset
  for (bs_kv_paged* p = h->caches; p; p = p->next) p->last_t = p->table_t = -2;
  return BS_OK;
}

void bs_destroy(bs_state* h) {
  if (!h) return;
  for (bs_kv_paged* p = h->caches; p; p = p->next) p->h = nullptr;  // orphaned
  (void)hipStreamSynchronize(h->stream);
  (void)hipFree(h->block);
  free(h);
}

int bs_verify_create(int32_t batch, int32_t k, int32_t vocab, int32_t logits_dtype,
                     void* hip_stream, bs_verify_state** out) {
  if (!out) return BS_EINVAL;
  *out = nullptr;
  if (batch < 1 || k < 1 || k > 64 || vocab < 1) return BS_EINVAL;
  if ((int64_t)batch * k > kMaxGridRows) return BS_EINVAL;
  if (logits_dtype != BS_F32 && logits_dtype != BS_BF16) return BS_EINVAL;
  bs_verify_state* h = (bs_verify_state*)calloc(1, sizeof(bs_verify_state));
  if (!h) return BS_ENOMEM;
  h->stream = (hipStream_t)hip_stream;
  if (hipGetDevice(&h->device) != hipSuccess) {
    free(h);
    return BS_EDEVICE;
  }
  h->B = batch;
  h->k = k;
  h->V = vocab;
  h->dtype = logits_dtype;
  // 16 logits per thread: measured faster than 32 or 64 per thread on the
  // verify shapes (more, shorter workgroups in flight)
  h->ept = 16;
  h->tile = kThreads * h->ept;
  h->tiles = (vocab + h->tile - 1) / h->tile;
  const size_t pt = (size_t)batch * k * h->tiles;
  if (hipMalloc(&h->block, 3 * align_up(pt * 4)) != hipSuccess) {
    (void)hipGetLastError();
    free(h);
    return BS_ENOMEM;
  }
  h->px = (float*)h->block;
  h->pv = (int*)((char*)h->block + align_up(pt * 4));
  h->pc = (int*)((char*)h->block + 2 * align_up(pt * 4));
  *out = h;
  return BS_OK;
}

int bs_verify_ex(bs_verify_state* h, const void* logits, int64_t row_stride_elems,
                 const int32_t* proposals, int32_t top_k, int32_t min_block,
                 int32_t* accept_len, int32_t* argmax, int32_t* prop_rank) {
  if (!h || !logits || !proposals || !accept_len || !argmax) return BS_EINVAL;
  if (row_stride_elems < h->V || top_k < 1 || min_block < 0 || min_block > h->k)
    return BS_EINVAL;
  return launch_verify(h->stream, h->dtype, h->B, h->k, h->V, h->tiles, logits,
                       row_stride_elems, proposals, top_k, min_block, accept_len, argmax,
                       prop_rank, h->px, h->pv, h->pc);
}

int bs_verify(bs_verify_state* h, const void* logits, int64_t row_stride_elems,
              const int32_t* proposals, int32_t* accept_len, int32_t* argmax) {
  return bs_verify_ex(h, logits, row_stride_elems, proposals, 1, 0, accept_len, argmax, nullptr);
}

int bs_verify_noalloc(void* hip_stream, const void* logits, int32_t logits_dtype, int32_t batch,
                      int32_t k, int32_t vocab, int64_t row_stride_elems,
                      const int32_t* proposals, int32_t* accept_len, int32_t* argmax) {
  if (!logits || !proposals || !accept_len || !argmax) return BS_EINVAL;
  if (batch < 1 || k < 1 || k > 64 || vocab < 1 || row_stride_elems < vocab) return BS_EINVAL;
  if ((int64_t)batch * k > kMaxGridRows) return BS_EINVAL;
  if (logits_dtype != BS_F32 && logits_dtype != BS_BF16) return BS_EINVAL;
  const int rows = batch * k;
  const int tiles = (vocab + kThreads * 16 - 1) / (kThreads * 16);
  const size_t part = align_up((size_t)rows * verify_segments_for(rows, tiles) * 4);
  if (2 * part > kScratchBytes) return BS_EINVAL;
  void* base = nullptr;
  const int rc = scratch_address(&base);
  if (rc != BS_OK) return rc;
  float* px = (float*)base;
  int* pv = (int*)((char*)base + part);
  return launch_verify((hipStream_t)hip_stream, logits_dtype, batch, k, vocab, tiles, logits,
                       row_stride_elems, proposals, 1, 0, accept_len, argmax, nullptr, px, pv,
                       nullptr);
}

void bs_verify_destroy(bs_verify_state* h) {
  if (!h) return;
  (void)hipStreamSynchronize(h->stream);
  (void)hipFree(h->block);
  free(h);
}

}  // extern "C"
