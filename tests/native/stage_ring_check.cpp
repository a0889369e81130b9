// CPU check of the staging ring's sequencing (paged_kv_attention_plan_amd/csrc/stage.h).
//
// A simulated GPU thread plays the upload kernel: it takes launched uploads in
// stream order, waits (a long kernel queued ahead of them), copies the staged
// bytes, then stores the upload's sequence number into each of its workgroups'
// flags in a random order.  The host side runs the same acquire / fill /
// launched sequence as pkv_plan_upload.  Every upload must read exactly the
// bytes staged for it.
//
// usage: stage_ring_check MODE   with MODE one of
//   ring     guarded uploads; exit 0 iff every upload read its own bytes and
//            at least one acquire had to wait
//   unguarded  the host skips acquire() (writes the next buffer at once); the
//            check is expected to see an overwritten upload and exit 3
//   timeout  a reader that never finishes: acquire must fail after the timeout
//   stale    flags holding the previous sequence number do not free a buffer
#include <algorithm>
#include <atomic>
#include <chrono>
#include <condition_variable>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <deque>
#include <mutex>
#include <random>
#include <thread>
#include <vector>

#include "stage.h"

using namespace std::chrono;

namespace {

constexpr size_t kCap = 4096;
constexpr int kFlags = 8;

struct Job {
  pkv::Stage* stage;
  uint32_t seq;
  int readers;
  int step;
};

struct FakeGpu {
  std::mutex mu;
  std::condition_variable cv;
  std::deque<Job> q;
  bool done = false;
  std::vector<std::vector<unsigned char>> read;  // bytes each step's upload read
  microseconds head_delay{0};                    // a long kernel ahead of the first upload

  void run() {
    std::mt19937 rng(7);
    bool first = true;
    for (;;) {
      Job j;
      {
        std::unique_lock<std::mutex> lk(mu);
        cv.wait(lk, [&] { return done || !q.empty(); });
        if (q.empty()) return;
        j = q.front();
        q.pop_front();
      }
      if (first) std::this_thread::sleep_for(head_delay);
      first = false;
      std::vector<unsigned char> buf(kCap);
      std::memcpy(buf.data(), j.stage->host, kCap);  // the kernel's reads
      read[j.step] = buf;
      std::vector<int> order(j.readers);
      for (int i = 0; i < j.readers; ++i) order[i] = i;
      std::shuffle(order.begin(), order.end(), rng);
      for (int i : order) {
        std::this_thread::sleep_for(microseconds(50));
        std::atomic_thread_fence(std::memory_order_release);
        j.stage->flags()[i] = j.seq;
      }
    }
  }
};

void alloc(pkv::Stage& s) {
  s.host = std::calloc(1, kCap + kFlags * sizeof(uint32_t));
  s.cap = kCap;
  for (int i = 0; i < kFlags; ++i) s.flags()[i] = s.seq;
}

int ring_mode(bool guarded) {
  pkv::StageRing ring;
  alloc(ring.stage[0]);
  alloc(ring.stage[1]);
  constexpr int kSteps = 12;
  FakeGpu gpu;
  gpu.read.resize(kSteps);
  gpu.head_delay = milliseconds(30);
  std::thread t([&] { gpu.run(); });
  for (int step = 0; step < kSteps; ++step) {
    pkv::Stage* s = guarded ? ring.acquire(seconds(10)) : &ring.stage[ring.next];
    if (s == nullptr) {
      std::printf("step %d: acquire timed out\n", step);
      return 1;
    }
    std::memset(s->host, 0x10 + step, kCap);  // this step's plan
    const int readers = 1 + step % kFlags;
    const uint32_t seq = ring.next_seq();
    {
      std::lock_guard<std::mutex> lk(gpu.mu);
      gpu.q.push_back(Job{s, seq, readers, step});
    }
    gpu.cv.notify_one();
    ring.launched(readers);
  }
  {
    std::lock_guard<std::mutex> lk(gpu.mu);
    gpu.done = true;
  }
  gpu.cv.notify_one();
  t.join();
  int bad = 0;
  for (int step = 0; step < kSteps; ++step)
    for (size_t i = 0; i < kCap; ++i)
      if (gpu.read[step][i] != (unsigned char)(0x10 + step)) {
        std::printf("step %d read bytes of another step (0x%02x)\n", step, gpu.read[step][i]);
        ++bad;
        break;
      }
  std::printf("uploads %lld waits %lld wait_us %.1f bad %d\n", (long long)ring.uploads,
              (long long)ring.waits, ring.wait_ns / 1e3, bad);
  if (bad) return 3;
  if (ring.uploads != kSteps) return 1;
  if (guarded && ring.waits == 0) {
    std::printf("no acquire waited: the guard was not exercised\n");
    return 1;
  }
  return 0;
}

int timeout_mode() {
  pkv::StageRing ring;
  alloc(ring.stage[0]);
  alloc(ring.stage[1]);
  if (ring.acquire(seconds(1)) == nullptr) return 1;
  ring.launched(4);  // four readers that never store their flags
  if (ring.acquire(seconds(1)) == nullptr) return 1;  // the other buffer is free
  ring.launched(0);  // an upload of nothing has no reader to wait for
  const auto t0 = steady_clock::now();
  pkv::Stage* s = ring.acquire(milliseconds(20));
  const double ms = duration<double, std::milli>(steady_clock::now() - t0).count();
  std::printf("acquire of a never-finished buffer: %s after %.1f ms\n", s ? "returned" : "failed", ms);
  if (s != nullptr || ms < 20.0 || ring.waits != 1) return 1;
  // three of four readers done: still busy
  pkv::Stage& b = ring.stage[0];
  for (int i = 0; i < 3; ++i) b.flags()[i] = b.seq;
  if (ring.acquire(milliseconds(5)) != nullptr) return 1;
  b.flags()[3] = b.seq;
  if (ring.acquire(milliseconds(5)) == nullptr) return 1;
  return 0;
}

int stale_mode() {
  pkv::StageRing ring;
  alloc(ring.stage[0]);
  alloc(ring.stage[1]);
  for (int k = 0; k < 2; ++k) {  // two completed uploads through buffer 0
    pkv::Stage* s = ring.acquire(seconds(1));
    if (s != &ring.stage[0]) return 1;
    const uint32_t seq = ring.next_seq();
    ring.launched(2);
    s->flags()[0] = s->flags()[1] = seq;
    if (ring.acquire(seconds(1)) != &ring.stage[1]) return 1;
    ring.launched(0);
  }
  // a third upload whose readers have not run: the flags still hold the last seq
  if (ring.acquire(seconds(1)) != &ring.stage[0]) return 1;
  ring.launched(2);
  if (ring.acquire(seconds(1)) != &ring.stage[1]) return 1;
  ring.launched(0);
  if (ring.acquire(milliseconds(5)) != nullptr) {
    std::printf("a flag from the previous upload freed the buffer\n");
    return 1;
  }
  return 0;
}

}  // namespace

int main(int argc, char** argv) {
  const char* mode = argc > 1 ? argv[1] : "ring";
  if (!std::strcmp(mode, "ring")) return ring_mode(true);
  if (!std::strcmp(mode, "unguarded")) return ring_mode(false);
  if (!std::strcmp(mode, "timeout")) return timeout_mode();
  if (!std::strcmp(mode, "stale")) return stale_mode();
  return 2;
}
