// Host-threaded model of a single-launch GroupNorm protocol (statistics and
// normalisation in one launch), to find on the CPU which forms of it can
// fail to finish. Work-groups are threads that take items from one atomic
// queue; a statistics item adds its chunk's partial sums and bumps its
// frame's counter, the last finisher reduces the frame's partials and
// raises the frame's flag; a normalisation item of a frame waits for that
// flag with a bounded poll. Item order: statistics chunks of frame t, then
// normalisation chunks of frame t - lag.
//
// usage: model VARIANT FRAMES PIXELS CHUNK_PX LAG WORKERS BOUND [STATS_US]
//   STATS_US: microseconds a statistics item takes (0 by default), so that
//   normalisation items can be taken while their frame is still in flight,
//   as work-groups running side by side on a GPU do
//   VARIANT: ok          the protocol as described
//            pixel_target the counter counts pixels but its target is
//                         chunks * chunk_px (a ragged last chunk never
//                         completes it)
//            hoisted     the poll reads the flag once (a plain load the
//                         compiler may hoist, or a cached line never refreshed)
//            lag_short   normalisation items are emitted only while t < frames
//            norm_first  normalisation chunks of frame t precede its statistics
// Prints: finished, timeouts (bounded waits that ran out), frames normalised.
#include <algorithm>
#include <atomic>
#include <chrono>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <thread>
#include <vector>

struct Item { int kind, frame, chunk; };   // kind 0 = statistics, 1 = normalisation

int main(int argc, char** argv) {
  if (argc != 8 && argc != 9) return 2;
  const int stats_us = argc == 9 ? atoi(argv[8]) : 0;
  const std::string v = argv[1];
  const int frames = atoi(argv[2]), P = atoi(argv[3]), chunk_px = atoi(argv[4]);
  const int lag = atoi(argv[5]), workers = atoi(argv[6]);
  const long bound = atol(argv[7]);
  const int chunks = (P + chunk_px - 1) / chunk_px;

  std::vector<Item> q;
  const int last_t = v == "lag_short" ? frames - 1 : frames - 1 + lag;
  for (int t = 0; t <= last_t; ++t) {
    if (v == "norm_first" && t < frames)
      for (int c = 0; c < chunks; ++c) q.push_back({1, t, c});
    if (t < frames)
      for (int c = 0; c < chunks; ++c) q.push_back({0, t, c});
    if (v != "norm_first" && t - lag >= 0 && t - lag < frames)
      for (int c = 0; c < chunks; ++c) q.push_back({1, t - lag, c});
  }

  std::atomic<int> head{0};
  std::vector<std::atomic<long>> count(frames);
  std::vector<std::atomic<int>> flag(frames);
  std::vector<std::atomic<int>> normalised(frames * chunks);
  for (auto& c : count) c = 0;
  for (auto& f : flag) f = 0;
  for (auto& n : normalised) n = 0;
  std::atomic<long> timeouts{0};

  auto work = [&]() {
    for (;;) {
      const int i = head.fetch_add(1);
      if (i >= (int)q.size()) return;
      const Item it = q[i];
      if (it.kind == 0) {
        if (stats_us) std::this_thread::sleep_for(std::chrono::microseconds(stats_us));
        const int px = std::min(chunk_px, P - it.chunk * chunk_px);
        if (v == "pixel_target") {
          const long before = count[it.frame].fetch_add(px, std::memory_order_acq_rel);
          if (before + px == (long)chunks * chunk_px) flag[it.frame].store(1, std::memory_order_release);
        } else {
          const long before = count[it.frame].fetch_add(1, std::memory_order_acq_rel);
          if (before + 1 == chunks) flag[it.frame].store(1, std::memory_order_release);
        }
      } else {
        long n = 0;
        if (v == "hoisted") {
          const int seen = flag[it.frame].load(std::memory_order_relaxed);   // read once
          while (!seen && n < bound) { ++n; std::this_thread::yield(); }
        } else {
          while (!flag[it.frame].load(std::memory_order_acquire) && n < bound) {
            ++n;
            std::this_thread::yield();
          }
        }
        if (n >= bound) timeouts.fetch_add(1);
        normalised[it.frame * chunks + it.chunk] = 1;
      }
    }
  };
  std::vector<std::thread> th;
  for (int w = 0; w < workers; ++w) th.emplace_back(work);
  for (auto& t : th) t.join();
  int done = 0;
  for (int f = 0; f < frames; ++f) {
    bool all = true;
    for (int c = 0; c < chunks; ++c) all = all && normalised[f * chunks + c];
    done += all;
  }
  printf("finished timeouts=%ld frames_normalised=%d of %d items=%zu chunks=%d\n",
         timeouts.load(), done, frames, q.size(), chunks);
  return 0;
}
