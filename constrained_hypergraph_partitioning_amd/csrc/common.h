// Internal declarations shared by the host orchestration and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <string>
#include <vector>

#include "chp.h"

typedef uint32_t u32;
typedef uint64_t u64;
typedef int64_t i64;
typedef int32_t i32;

#define NONE32 0xFFFFFFFFu
#define FX_SHIFT 40

// Error-flag bits raised by kernels into ctx->flags[0] (atomicOr); the host
// maps them to a return code by precedence EINVAL > EOVERFLOW > EINFEASIBLE.
#define FLAG_EINVAL 1u
#define FLAG_EOVERFLOW 2u
#define FLAG_EINFEASIBLE 4u
#define FLAG_ECYCLE 8u
#define FLAG_LONGCHAIN 16u  // a handshake walk hit its step limit (host falls back)

// Launch geometry
#define GRID_STRIDE_BLOCKS 4096  // grid of the persistent work-list kernels

struct TimingRec {
  const char *name;
  hipEvent_t a, b;
};

struct TimingSum {
  const char *name;
  u64 launches;
  double total_ms;
};

struct chp_ctx {
  hipStream_t stream = nullptr;
  chp_alloc_fn alloc = nullptr;
  chp_free_fn free_fn = nullptr;
  void *user = nullptr;
  int device = 0;
  u32 n_cu = 256;          // compute units of the device
  std::string err;
  u32 *flags = nullptr;    // device: [0] error flags, [1..63] small counters
  char *arena = nullptr;   // device scratch reused by every call
  size_t arena_cap = 0, arena_top = 0;
  u64 *pinned = nullptr;   // host pinned staging (64 words), mapped
  u32 *pinned_dev = nullptr;  // its device address
  u64 batch_entries = 0;      // neighbour entries per rating batch (0 = default)
  u64 last_nb_built = 0;      // entries the last batched rating built
  u32 last_batches = 0;       // and its number of batches
  u32 last_inc_nodes = 0;     // nodes it rated straight from the incidence
  u64 inc_min_visits = 0;     // incident pins that send a node there (0 = default)
  u32 inc_hash_keys = 0;      // keys a sparse window there may claim (0 = all it holds)
  u32 inc_bins = 0;           // CHP_INC_BINS_32 (default) or CHP_INC_BINS_64 there
  u32 matching = 0;           // CHP_MATCH_HANDSHAKE or CHP_MATCH_OPTIMAL
  u32 move_order = 0;         // CHP_ORDER_CHAINS or CHP_ORDER_GAIN
  u64 *dsmall = nullptr;   // device small buffer (64 words)
  char *fixed_scratch = nullptr;  // this device's copy of the library's fixed scratch array
  int timing = 0;
  std::string timing_prefix;  // time only kernels whose name starts with it ("" = all)
  std::vector<TimingRec> pending;
  std::vector<hipEvent_t> free_events;
  std::vector<TimingSum> sums;
};

// ---- host helpers (api.hip) ----------------------------------------------
void *ctx_alloc(chp_ctx *c, size_t bytes);
void ctx_free(chp_ctx *c, void *p);
void timing_begin(chp_ctx *c, const char *name, hipEvent_t *a, hipEvent_t *b);
inline bool timing_wanted(const chp_ctx *c, const char *name) {
  return c->timing_prefix.empty() ||
         c->timing_prefix.compare(0, std::string::npos, name, c->timing_prefix.size()) == 0;
}
void timing_end(chp_ctx *c, const char *name, hipEvent_t a, hipEvent_t b);

// Launch helper that brackets the launch with events when timing is on.
#define CHP_LAUNCH(ctx, name, kern, grid, block, shmem, ...)                         \
  do {                                                                               \
    hipEvent_t ev_a_ = nullptr, ev_b_ = nullptr;                                     \
    const bool timed_ = (ctx)->timing && timing_wanted((ctx), (name));               \
    if (timed_) timing_begin((ctx), (name), &ev_a_, &ev_b_);                         \
    hipLaunchKernelGGL(kern, dim3(grid), dim3(block), shmem, (ctx)->stream,          \
                       __VA_ARGS__);                                                 \
    if (timed_) timing_end((ctx), (name), ev_a_, ev_b_);                             \
  } while (0)

static inline u32 grid_for(u64 n, u32 block) {
  u64 g = (n + block - 1) / block;
  if (g == 0) g = 1;
  if (g > 0x7FFFFFFFull) g = 0x7FFFFFFFull;
  return (u32)g;
}

// grid of 256-thread blocks giving one wave per item (capped; kernels stride)
static inline u32 waves_grid(u64 items) {
  u64 g = (items + 3) / 4;
  if (g > 16384) g = 16384;
  if (g == 0) g = 1;
  return (u32)g;
}

// ---- kernel launchers (defined in the k_*.hip files) ----------------------
// scan.hip: out[i] = sum_{j<i} in[j] for i in [0,n], out has n+1 entries.
void scan_u32_to_i64(chp_ctx *c, const u32 *in, i64 *out, u64 n, i64 *tmp);
void scan_i64(chp_ctx *c, const i64 *in, i64 *out, u64 n, i64 *tmp);
size_t scan_tmp_words(u64 n);
