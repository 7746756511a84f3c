// Instantiations of the ReplaySSM window kernel for state size n = 256: the
// append (T = 0 here), the verify of T = 1..8 drafts and the fused front-end,
// head dims 64 and 128
// (own translation unit so the kernel variants compile in parallel).
#include "replay.hpp"

namespace rssm_host {

int launch_replay_n256(int T, int D, const ReplayParams& p, int B, void* stream) {
  switch (T) {
    case 0: return D == 64 ? launch_window<64, 1, true, false, 256>(p, B, stream)
                           : launch_window<128, 1, true, false, 256>(p, B, stream);
    case 1: return D == 64 ? launch_window<64, 1, false, false, 256>(p, B, stream)
                           : launch_window<128, 1, false, false, 256>(p, B, stream);
    case 2: return D == 64 ? launch_window<64, 2, false, false, 256>(p, B, stream)
                           : launch_window<128, 2, false, false, 256>(p, B, stream);
    case 3: return D == 64 ? launch_window<64, 3, false, false, 256>(p, B, stream)
                           : launch_window<128, 3, false, false, 256>(p, B, stream);
    case 4: return D == 64 ? launch_window<64, 4, false, false, 256>(p, B, stream)
                           : launch_window<128, 4, false, false, 256>(p, B, stream);
    case 5: return D == 64 ? launch_window<64, 5, false, false, 256>(p, B, stream)
                           : launch_window<128, 5, false, false, 256>(p, B, stream);
    case 6: return D == 64 ? launch_window<64, 6, false, false, 256>(p, B, stream)
                           : launch_window<128, 6, false, false, 256>(p, B, stream);
    case 7: return D == 64 ? launch_window<64, 7, false, false, 256>(p, B, stream)
                           : launch_window<128, 7, false, false, 256>(p, B, stream);
    case 8: return D == 64 ? launch_window<64, 8, false, false, 256>(p, B, stream)
                           : launch_window<128, 8, false, false, 256>(p, B, stream);
    default: return RSSM_ENOTSUP;
  }
}

int launch_replay_conv_n256(int D, const ReplayParams& p, int B, void* stream) {
  return D == 64 ? launch_window<64, 1, true, true, 256>(p, B, stream) : launch_window<128, 1, true, true, 256>(p, B, stream);
}

}  // namespace rssm_host
