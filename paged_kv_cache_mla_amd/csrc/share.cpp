// CPU / GPU share policy: the balance of the two engines' step latencies and the routing of
// tokens leaving the GPU staging window.
//
// "Physically Partitioned KVCache Format for CPU-GPU Load Balancing in MoE Inference":
//   §5.1  the CPU takes the oldest r * L tokens of a sequence, the GPU the newest;
//   §5.2  Eq. 1: T_CPU(r) = r A L + C_CPU and T_GPU(r) = (1 - r) B L + C_GPU;
//   §5.3  Eq. 2: their balance r(L), clamped to [0, 1], converging to p = B / (A + B); B is
//         calibrated once, A is re-estimated online from a sliding average of the CPU's
//         per-step latency; evicted batches are routed so that the cumulative share follows
//         r(L), moving toward p by at most one batch's worth (D / L) each time.
// Pure C++17 with no HIP dependency; the controller is a small struct owned by the caller.

#include <cmath>
#include <cstdint>
#include <new>
#include <string>
#include <vector>

#include "pool_internal.h"

struct kvattn_share_ctl {
  kvattn_share_model model;  // cpu_cost is the current A
  int32_t window;
  std::vector<double> t_ring, n_ring;
  int32_t held = 0, next = 0;
  bool admitted = false;
  int64_t placed = 0, cpu = 0, cpu_batches = 0, batches = 0;
};

namespace kvattn {
namespace {

bool model_ok(const kvattn_share_model* m) {
  return m && std::isfinite(m->cpu_cost) && std::isfinite(m->gpu_cost) &&
         std::isfinite(m->cpu_fixed) && std::isfinite(m->gpu_fixed) && m->cpu_cost >= 0 &&
         m->gpu_cost >= 0 && m->cpu_cost + m->gpu_cost > 0;
}

// Eq. 2; L > 0.
double optimum(const kvattn_share_model& m, double L) {
  const double ab = m.cpu_cost + m.gpu_cost;
  const double r = m.gpu_cost / ab + (m.gpu_fixed - m.cpu_fixed) / (ab * L);
  return std::fmin(1.0, std::fmax(0.0, r));
}

}  // namespace

// CPU tokens the admission of `prefill_tokens` gives (whole blocks, nearest, at most the
// whole blocks of the prefill), without admitting: -1 if the controller is already admitted.
int64_t share_admit_tokens(const kvattn_share_ctl* ctl, int64_t prefill_tokens,
                           int64_t block_tokens) {
  if (ctl->admitted) return -1;
  if (prefill_tokens <= 0) return 0;
  const double r = optimum(ctl->model, (double)prefill_tokens);
  const int64_t whole = prefill_tokens / block_tokens;
  int64_t blocks = (int64_t)std::llround(r * (double)prefill_tokens / (double)block_tokens);
  if (blocks > whole) blocks = whole;
  return blocks * block_tokens;
}

}  // namespace kvattn

using kvattn::set_error;

extern "C" {

kvattn_status kvattn_share_optimum(const kvattn_share_model* model, double placed_len,
                                   double* r_out) {
  if (!kvattn::model_ok(model) || !r_out)
    return set_error(KVATTN_E_INVAL, "share_optimum: null pointer or invalid cost model");
  if (!std::isfinite(placed_len) || placed_len <= 0)
    return set_error(KVATTN_E_INVAL, "share_optimum: placed length must be finite and > 0");
  *r_out = kvattn::optimum(*model, placed_len);
  return KVATTN_OK;
}

kvattn_status kvattn_share_fit(const double* tokens, const double* seconds, int32_t count,
                               double* slope, double* intercept) {
  if (!tokens || !seconds || !slope || !intercept || count < 2)
    return set_error(KVATTN_E_INVAL, "share_fit: null pointer or fewer than 2 points");
  // centred sums: slope = S_xy / S_xx, intercept = mean_y - slope * mean_x
  double mx = 0, my = 0;
  for (int32_t i = 0; i < count; ++i) {
    if (!std::isfinite(tokens[i]) || !std::isfinite(seconds[i]))
      return set_error(KVATTN_E_INVAL, "share_fit: non-finite point");
    mx += tokens[i];
    my += seconds[i];
  }
  mx /= count;
  my /= count;
  double sxx = 0, sxy = 0;
  for (int32_t i = 0; i < count; ++i) {
    const double dx = tokens[i] - mx;
    sxx += dx * dx;
    sxy += dx * (seconds[i] - my);
  }
  if (!(sxx > 0)) return set_error(KVATTN_E_INVAL, "share_fit: all token counts are equal");
  *slope = sxy / sxx;
  *intercept = my - *slope * mx;
  return KVATTN_OK;
}

kvattn_status kvattn_share_ctl_create(const kvattn_share_model* model, int32_t window,
                                      kvattn_share_ctl** out) {
  if (!out) return set_error(KVATTN_E_INVAL, "share_ctl_create: null output");
  *out = nullptr;
  if (!kvattn::model_ok(model))
    return set_error(KVATTN_E_INVAL, "share_ctl_create: invalid cost model");
  if (window < 1 || window > 65536)
    return set_error(KVATTN_E_INVAL, "share_ctl_create: window must be in [1, 65536]");
  kvattn_share_ctl* c = new (std::nothrow) kvattn_share_ctl();
  if (!c) return set_error(KVATTN_E_INVAL, "share_ctl_create: out of host memory");
  c->model = *model;
  c->window = window;
  c->t_ring.assign(window, 0.0);
  c->n_ring.assign(window, 0.0);
  *out = c;
  return KVATTN_OK;
}

void kvattn_share_ctl_free(kvattn_share_ctl* ctl) { delete ctl; }

kvattn_status kvattn_share_admit(kvattn_share_ctl* ctl, int64_t prefill_tokens,
                                 int64_t block_tokens, int64_t* cpu_tokens) {
  if (!ctl || !cpu_tokens) return set_error(KVATTN_E_INVAL, "share_admit: null pointer");
  if (ctl->admitted) return set_error(KVATTN_E_STATE, "share_admit: already admitted");
  if (prefill_tokens < 0 || block_tokens < 1)
    return set_error(KVATTN_E_INVAL, "share_admit: prefill_tokens < 0 or block_tokens < 1");
  const int64_t c = kvattn::share_admit_tokens(ctl, prefill_tokens, block_tokens);
  ctl->admitted = true;
  ctl->placed = prefill_tokens;
  ctl->cpu = c;
  *cpu_tokens = c;
  return KVATTN_OK;
}

kvattn_status kvattn_share_observe(kvattn_share_ctl* ctl, double cpu_seconds, double cpu_tokens) {
  if (!ctl) return set_error(KVATTN_E_INVAL, "share_observe: null controller");
  if (!ctl->admitted) return set_error(KVATTN_E_STATE, "share_observe: not admitted");
  if (!std::isfinite(cpu_seconds) || !std::isfinite(cpu_tokens) || cpu_seconds < 0 ||
      cpu_tokens < 0)
    return set_error(KVATTN_E_INVAL, "share_observe: sample must be finite and >= 0");
  ctl->t_ring[ctl->next] = cpu_seconds;
  ctl->n_ring[ctl->next] = cpu_tokens;
  ctl->next = (ctl->next + 1) % ctl->window;
  if (ctl->held < ctl->window) ++ctl->held;
  return KVATTN_OK;
}

kvattn_status kvattn_share_route(kvattn_share_ctl* ctl, int64_t batch_tokens, int32_t* to_cpu) {
  if (!ctl || !to_cpu) return set_error(KVATTN_E_INVAL, "share_route: null pointer");
  if (!ctl->admitted) return set_error(KVATTN_E_STATE, "share_route: not admitted");
  if (batch_tokens < 1) return set_error(KVATTN_E_INVAL, "share_route: batch_tokens < 1");
  if (ctl->held == ctl->window) {
    // sums recomputed from the ring each time (no running-sum drift), oldest sample first
    double st = 0, sn = 0;
    for (int32_t j = 0; j < ctl->window; ++j) {
      const int32_t i = (ctl->next + j) % ctl->window;
      st += ctl->t_ring[i];
      sn += ctl->n_ring[i];
    }
    if (sn > 0) {
      const double a = (st - ctl->window * ctl->model.cpu_fixed) / sn;
      if (a > 0 && std::isfinite(a)) ctl->model.cpu_cost = a;
    }
  }
  const int64_t after = ctl->placed + batch_tokens;
  const double target = kvattn::optimum(ctl->model, (double)after) * (double)after;
  const bool cpu = (double)ctl->cpu + 0.5 * (double)batch_tokens < target;
  if (cpu) {
    ctl->cpu += batch_tokens;
    ++ctl->cpu_batches;
  }
  ++ctl->batches;
  ctl->placed = after;
  *to_cpu = cpu ? 1 : 0;
  return KVATTN_OK;
}

kvattn_status kvattn_share_get_state(const kvattn_share_ctl* ctl, kvattn_share_state* out) {
  if (!ctl || !out) return set_error(KVATTN_E_INVAL, "share_get_state: null pointer");
  out->placed_tokens = ctl->placed;
  out->cpu_tokens = ctl->cpu;
  out->cpu_batches = ctl->cpu_batches;
  out->batches = ctl->batches;
  out->cpu_cost = ctl->model.cpu_cost;
  out->converged = ctl->model.gpu_cost / (ctl->model.cpu_cost + ctl->model.gpu_cost);
  out->target_share = ctl->placed > 0 ? kvattn::optimum(ctl->model, (double)ctl->placed) : 0.0;
  out->samples = ctl->held;
  return KVATTN_OK;
}

}  // extern "C"
