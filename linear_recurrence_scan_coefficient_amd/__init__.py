"""MI355X-native batched linear-recurrence scans for RL credit assignment."""
