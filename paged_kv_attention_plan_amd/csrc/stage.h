// The page-locked staging ring of plan uploads (kv.plan PinnedIndexRing: a
// set of pinned host buffers reused round-robin, each rewritten only after the
// copy that last read it has finished; attn.dense force_double_buffer: the
// plan of step N+1 must not overwrite a buffer step N still reads).
//
// Host-only code (no HIP calls), so that its sequencing can be tested on the
// CPU against a simulated reader.
#pragma once

#include <chrono>
#include <cstddef>
#include <cstdint>
#include <thread>

namespace pkv {

// One buffer of the ring: [0, cap) holds the serialised plan, followed by one
// completion flag per reading workgroup.  Each workgroup of the upload that
// reads the buffer stores the upload's sequence number into its flag when its
// reads are done; the buffer may be rewritten once every flag holds it.
struct Stage {
  void* host = nullptr;
  void* dev = nullptr;  // the same memory as seen by the GPU
  size_t cap = 0;
  uint32_t seq = 0;     // sequence number of the last upload from this buffer
  int n_flags = 0;      // workgroups of that upload
  bool pending = false;
  volatile uint32_t* flags() const {
    return reinterpret_cast<volatile uint32_t*>(static_cast<char*>(host) + cap);
  }
};

// Wait until every reader of the stage's last upload has stored its sequence
// number.  Spins, then yields; returns false after `timeout` (the reader
// counts as failed).  *waited is set when the readers were not done at the
// first look.
inline bool wait_stage(Stage& s, std::chrono::nanoseconds timeout, bool* waited = nullptr) {
  if (waited != nullptr) *waited = false;
  if (!s.pending) return true;
  const auto t0 = std::chrono::steady_clock::now();
  for (int spin = 0;; ++spin) {
    int i = 0;
    while (i < s.n_flags && s.flags()[i] == s.seq) ++i;
    if (i == s.n_flags) {
      s.pending = false;
      return true;
    }
    if (waited != nullptr) *waited = true;
    if (spin >= 64) {
      std::this_thread::yield();
      if ((spin & 255) == 0 && std::chrono::steady_clock::now() - t0 > timeout) return false;
    }
  }
}

// Depth-2 ring.  An upload takes the next buffer with acquire() (which waits
// for that buffer's previous readers), fills it, launches its readers with
// sequence number next_seq(), then calls launched() with their count.
struct StageRing {
  Stage stage[2];
  int next = 0;
  int64_t uploads = 0;   // launched() calls
  int64_t waits = 0;     // acquire() calls that found the buffer still being read
  int64_t wait_ns = 0;   // time spent in those waits

  Stage* acquire(std::chrono::nanoseconds timeout) {
    Stage& s = stage[next];
    bool waited = false;
    const auto t0 = std::chrono::steady_clock::now();
    const bool ok = wait_stage(s, timeout, &waited);
    if (waited) {
      ++waits;
      wait_ns += std::chrono::duration_cast<std::chrono::nanoseconds>(
                     std::chrono::steady_clock::now() - t0).count();
    }
    return ok ? &s : nullptr;
  }
  uint32_t next_seq() const { return stage[next].seq + 1; }
  // The buffer acquired last now has `readers` workgroups in flight that
  // will store next_seq() into its first `readers` flags.
  void launched(int readers) {
    Stage& s = stage[next];
    s.seq += 1;
    s.n_flags = readers;
    s.pending = true;
    next ^= 1;
    ++uploads;
  }
};

}  // namespace pkv
