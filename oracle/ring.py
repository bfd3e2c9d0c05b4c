"""List model of the sliding-window KV cache (test infrastructure only).

The pages: earlier segments' keys and values are carried in a cache
(orcarouter.ai, section "Die Schleife"); on one GPU only the last 18 latent
frames stay on the device and older ones are moved out ("Hy-Nomas auf einer RTX
4090", inferencekey.com, sections "Die Autoren betreiben es auf acht GPUs" and
"Das Single-GPU-Preset"; blog.authon.dev, "What Hy-Nomas is" and the
``sliding_window: past_frames: 18`` excerpt). Readings:

* the window holds whole latent frames, the most recent ``capacity`` of them,
  evicting the oldest first (one append may evict part of an earlier segment);
* a frame that was appended as the f-th frame of the session (f counted from 0)
  lives in physical slot f mod capacity while it is retained, so the retained
  frames always occupy slots [0, min(frames_written, capacity));
* an append of more than ``capacity`` frames keeps only its last ``capacity``.

The model is a plain list: no modular arithmetic is used to decide *which*
frames are retained, only to say where each retained frame is expected.
"""


class RingModel:
    def __init__(self, capacity_frames):
        if capacity_frames < 1:
            raise ValueError("capacity must be >= 1")
        self.capacity = capacity_frames
        self.frames = []            # list of (absolute frame index, payload)
        self.evicted = []           # frames that left the window, in order
        self.frames_written = 0

    def append(self, payloads):
        """Append frames in order; each payload is any per-frame object."""
        for p in payloads:
            self.frames.append((self.frames_written, p))
            self.frames_written += 1
            while len(self.frames) > self.capacity:
                self.evicted.append(self.frames.pop(0))

    def retained(self):
        """Retained (absolute index, payload) pairs, oldest first."""
        return list(self.frames)

    def valid_frames(self):
        return len(self.frames)

    def expected_slots(self):
        """dict: physical slot -> (absolute index, payload) for retained frames."""
        return {f % self.capacity: (f, p) for f, p in self.frames}
