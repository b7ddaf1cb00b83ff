// Host-only driver for the library's plan and argument validation (plan.cpp, pure C++), built
// with AddressSanitizer and UndefinedBehaviorSanitizer by tests/test_sanitize_cpu.py: it sweeps
// plan parameters (valid and invalid, up to 2^30-token contexts and 65536 sequences), checks
// arguments against each valid plan and resolves launch arguments, so that any out-of-range
// access or signed overflow in that host arithmetic aborts the run. Test infrastructure only.
#include <cstdio>
#include <cstring>

#include "skvd_internal.h"

int main() {
  using namespace skvd;
  char err[512];
  long ok = 0, refused = 0;
  const int heads[][2] = {{32, 8}, {8, 8}, {32, 16}, {64, 1}, {12, 4}, {5, 5}, {8, 3}};
  const int dims[] = {64, 128, 256, 512};
  const int pages[] = {1, 2, 16, 64, 1024, 3, 0};
  const int batches[] = {1, 32, 64, 65, 4096, 65536, 0};
  const int lens[] = {1, 63, 64, 2048, 2049, 131072, 262208, 1 << 30, 0};
  for (auto &hh : heads)
    for (int D : dims)
      for (int P : pages)
        for (int B : batches)
          for (int L : lens)
            for (int T = 1; T <= 9; T += 4)
              for (int dt = 0; dt < 4; ++dt)  // f16, int8, fp8, and one unknown value
                for (int sched = 0; sched < 3; ++sched) {
                  skvd_plan_params prm{};
                  prm.num_qo_heads = hh[0];
                  prm.num_kv_heads = hh[1];
                  prm.head_dim = D;
                  prm.page_size = P;
                  prm.max_batch = B;
                  prm.max_q_per_seq = T;
                  prm.max_kv_len = L;
                  prm.kv_dtype = dt;
                  prm.schedule = sched;
                  Plan p{};
                  if (make_plan(prm, 256, &p, err, sizeof err) != SKVD_OK) {
                    ++refused;
                    continue;
                  }
                  ++ok;
                  skvd_decode_args a{};
                  static char fake[64] __attribute__((aligned(256)));
                  a.q = a.k_pages = a.v_pages = a.o = fake;
                  a.page_table = a.kv_len = (const int32_t *)fake;
                  a.q_tok_stride = (int64_t)hh[0] * D;
                  a.q_head_stride = D;
                  a.page_stride = (int64_t)P * hh[1] * D;
                  a.tok_stride = (int64_t)hh[1] * D;
                  a.head_stride = D;
                  a.num_k_pages = a.num_v_pages = 1000;
                  if (dt == SKVD_KV_FP8_E4M3) a.k_scales = a.v_scales = fake;  // one f32 each
                  if (dt == SKVD_KV_I8_F16SCALE32) {
                    a.k_scales = a.v_scales = fake;
                    a.scale_page_stride = (int64_t)P * hh[1] * (D / 32);
                    a.scale_tok_stride = (int64_t)hh[1] * (D / 32);
                    a.scale_head_stride = D / 32;
                  }
                  a.table_stride = ((int64_t)L + P - 1) / P;
                  a.batch = B;
                  a.q_per_seq = T;
                  a.sm_scale = 0.1f;
                  check_args(p, &a, p.ws_bytes, err, sizeof err);
                  check_args(p, &a, 0, err, sizeof err);
                  LaunchArgs la;
                  fill_launch_args(p, a, fake, &la);
                }
  std::printf("plan driver: %ld plans, %ld refused\n", ok, refused);
  return ok > 0 ? 0 : 1;
}
